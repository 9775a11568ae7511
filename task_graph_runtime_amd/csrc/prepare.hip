// Weight preparation for batch > 1 graphs (mpk_prepare_weights in
// include/mpk.h): a one-time copy of every projection matrix into the block
// order the matrix-core tiles load (see packed_block in tasks.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

namespace mpk {

namespace {

// dst = src [N][K] (bf16, row-major) as blocks [ceil(N/16)][K/32][64][8]:
// 16-byte chunk c of dst is lane c % 64 of block c / 64, i.e. row
// 16 rb + lane % 16 at k 32 ks + 8 (lane / 16); rows past N are zero.  With
// `b` given the source is the 2N/2 interleave of a and b (row 2i of a's row
// i, row 2i + 1 of b's).
__global__ void __launch_bounds__(256) pack_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                   int64_t N, int64_t K, uint4* __restrict__ dst, int64_t nchunks) {
  const int64_t nks = K >> 5;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
    const int lane = (int)(c & 63);
    const int64_t blk = c >> 6;
    const int64_t rb = blk / nks, ks = blk - rb * nks;
    const int64_t row = rb * 16 + (lane & 15);
    const int64_t k = ks * 32 + (lane >> 4) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < N) {
      const uint16_t* src = b ? ((row & 1) ? b : a) + (row >> 1) * K : a + row * K;
      v = *reinterpret_cast<const uint4*>(src + k);
    }
    dst[c] = v;
  }
}

}  // namespace

// Bytes of the prepared copy of an [N][K] matrix (K a multiple of 32).
int64_t packed_bytes(int64_t N, int64_t K) { return ((N + 15) / 16) * 16 * K * 2; }

hipError_t launch_pack(const void* a, const void* b, int64_t N, int64_t K, void* dst, hipStream_t stream) {
  const int64_t nchunks = ((N + 15) / 16) * (K / 32) * 64;
  if (nchunks == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(4096, (nchunks + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(a),
                     static_cast<const uint16_t*>(b), N, K, static_cast<uint4*>(dst), nchunks);
  return hipGetLastError();
}

}  // namespace mpk
