// Rotary position embedding for the chunk-recurrent layer: queries and keys are
// rotated by their absolute positions before keys enter the paged cache (chunk
// position t0 + i, gist.science explainer of OOMB, 2.A: the chunks of one sequence keep
// their global positions). Convention: pairs (d, d + D/2) of head dimension D,
//   y_d       = x_d cos a - x_{d+D/2} sin a,   y_{d+D/2} = x_{d+D/2} cos a + x_d sin a,
//   a = p * theta^(-2d/D)  (p the absolute position), inverse: a -> -a.
// The angle and its sine and cosine are taken in fp64 (at million-token positions an
// fp32 product would be off by a tenth of a radian), once per (token, pair); the
// rotation itself is fp32 and shared by every head; the result is rounded once to the
// tensor's dtype. Elementwise and HBM-bound.
#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  const int half = a.D / 2;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (token, pair)
  if (item >= static_cast<int64_t>(a.n_tok) * half) return;
  const int i = static_cast<int>(item / half), j = static_cast<int>(item % half);
  const double inv_freq = pow(static_cast<double>(a.theta), -2.0 * j / a.D);
  const double ang = static_cast<double>(a.pos0 + i) * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float c = static_cast<float>(cd), s = static_cast<float>(a.inverse ? -sd : sd);
  const T* x = static_cast<const T*>(a.x);
  T* y = static_cast<T*>(a.y);
  for (int h = 0; h < a.n_heads; ++h) {
    const int64_t xo = h * a.x_hs + static_cast<int64_t>(i) * a.x_ts + j;
    const int64_t yo = h * a.y_hs + static_cast<int64_t>(i) * a.y_ts + j;
    const float lo = to_f32(x[xo]), hi = to_f32(x[xo + half]);
    y[yo] = from_f32<T>(lo * c - hi * s);
    y[yo + half] = from_f32<T>(hi * c + lo * s);
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  const int64_t items = static_cast<int64_t>(a.n_tok) * (a.D / 2);
  const dim3 grid(static_cast<unsigned>((items + 255) / 256));
  if (a.dtype == 0) OOMB_LAUNCH("rope", rope_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else OOMB_LAUNCH("rope", rope_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
