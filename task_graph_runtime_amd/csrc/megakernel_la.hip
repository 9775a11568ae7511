// The persistent kernel of the paged lookahead (build parameter weight_preload
// = 3): the same runtime and task bodies as megakernel.hip, compiled as a
// kernel of its own (mpk_megakernel_la) so that the option leaves the default
// kernel's code as it is.  See worker_loop in megakernel.hip.
#define MPK_LA 1
#include "megakernel.hip"
