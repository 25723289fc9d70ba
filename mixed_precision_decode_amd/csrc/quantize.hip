// Per-token asymmetric INT4/INT2 quantization of fp16 rows.
//
// velog notes "No Token Left Behind ...", Key contributions 1) (per-token
// asymmetric quantization of the retained tokens) and 2), additional notes
// (group = half the head dimension); paperlayer summary of arXiv 2402.18096,
// section 3.2.
//
// One row of d channels is handled by d/8 lanes (16 bytes of fp16 each);
// a 256-thread block covers 256/(d/8) rows per step and strides over rows.
// HBM-bound: per row it reads 2d bytes and writes d*bits/8 + 4*d/group.
#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

template <int D, int BITS, int NL>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ rows,
                                                            int64_t n_rows,
                                                            uint8_t* __restrict__ codes,
                                                            uint32_t* __restrict__ sz) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPB = 256 / LPR;          // rows per block step
  constexpr int GROUPS = D / (8 * NL);    // groups per row
  constexpr int CB = D * BITS / 8;        // code bytes per row
  const int lane = threadIdx.x % LPR;
  const int64_t step = static_cast<int64_t>(gridDim.x) * RPB;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; r < n_rows; r += step) {
    const int64_t src = rows ? static_cast<int64_t>(rows[r]) : r;
    float v[8];
    load8(x + src * D + lane * 8, v);
    uint32_t szw;
    const uint32_t packed = quantize8<BITS, NL>(v, &szw);
    store_codes8<BITS>(codes + r * CB, lane, packed);
    if (lane % NL == 0) sz[r * GROUPS + lane / NL] = szw;
  }
}

template <int D, int BITS, int NL>
static hipError_t launch_q(const uint16_t* x, const int32_t* rows, int64_t n_rows, uint8_t* codes,
                           uint16_t* sz, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  int64_t blocks = (n_rows + RPB - 1) / RPB;
  if (blocks > 65536) blocks = 65536;
  quantize_rows_kernel<D, BITS, NL><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      x, rows, n_rows, codes, reinterpret_cast<uint32_t*>(sz));
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, const int32_t* rows, int64_t n_rows, int d,
                                int group, int bits, uint8_t* codes, uint16_t* sz,
                                hipStream_t stream) {
  // NL = group / 8 lanes per group
#define MIKV_Q(D_, B_, G_)                                              \
  if (d == D_ && bits == B_ && group == G_)                             \
    return launch_q<D_, B_, G_ / 8>(x, rows, n_rows, codes, sz, stream);
  MIKV_Q(128, 4, 64) MIKV_Q(128, 4, 128) MIKV_Q(128, 2, 64) MIKV_Q(128, 2, 128)
  MIKV_Q(64, 4, 32) MIKV_Q(64, 4, 64) MIKV_Q(64, 2, 32) MIKV_Q(64, 2, 64)
#undef MIKV_Q
  return hipErrorInvalidValue;
}

}  // namespace mikv
