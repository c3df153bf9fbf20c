// Input side of the model, fused: token embedding scaled by sqrt(d_model)
// plus the sinusoidal positional encoding, for gfx950 (bf16 or fp32):
//
//   out[b][p][j] = E[tokens[b][p]][j] * sqrt(d_model) + PE(pos0 + p, j)
//   PE(pos, 2i) = sin(pos * w_i),  PE(pos, 2i + 1) = cos(pos * w_i),
//   w_i = 10000^(-2i / d_model)
//
// (devpress.csdn.net "【深度学习】Transformer", section 4, equation (4.1), Table
// 4.1 and the worked example that scales the input by sqrt(d_model) before
// adding the encoding; hex4c59.cc "读懂 Attention Is All You Need", section
// "没有循环，模型怎样知道词序？": embedding row looked up by token id, times
// sqrt(d_model), plus the encoding.)
//
// One workgroup per (position, group of batch rows): the encoding depends on
// the position only, so each thread evaluates it once for its 16-byte chunk
// of the row -- frequency and angle in double precision (the angle reaches
// pos radians, where a single-precision argument would already be off by
// pos * 2^-24), reduced to one turn before a single-precision sine and
// cosine -- and reuses it for every batch row of the group.
// The embedding rows are gathered with 16-byte loads, all of a group's rows
// issued before the first use.  Bandwidth-bound: per token 2 d (or 4 d)
// bytes gathered and written.  A token id outside [0, vocab) produces a row
// of NaN and reads nothing.
#include <math.h>

#include "device.h"

namespace mha {
namespace {

using namespace dev;

constexpr int kRowsPerGroup = 8;  // batch rows per workgroup

constexpr double kLog2_10000 = 13.287712379549449;        // log2(10000)
constexpr double kInv2Pi = 0.15915494309189535;           // 1 / (2 pi)
constexpr double k2PiHi = 6.283185307179586;              // 2 pi rounded to double
constexpr double k2PiLo = 2.4492935982947064e-16;         // 2 pi - k2PiHi

template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

template <typename T>
__global__ __launch_bounds__(256) void embed_positional_kernel(const EmbedArgs a) {
  constexpr int N = Vec<T>::N;
  typedef typename Vec<T>::type VT;
  typedef float FV __attribute__((ext_vector_type(N)));
  const int p = blockIdx.x;
  const int b0 = blockIdx.y * kRowsPerGroup;
  const int rows = min(kRowsPerGroup, a.B - b0);
  const int chunks = a.d / N;
  const double pos = (double)a.pos0 + (double)p;
  const float scale = (float)sqrt((double)a.d);

  int tok[kRowsPerGroup];
#pragma unroll
  for (int r = 0; r < kRowsPerGroup; ++r) tok[r] = r < rows ? a.tokens[(int64_t)(b0 + r) * a.n + p] : 0;

  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    // The gathers go out first; the encoding is evaluated while they are in
    // flight.
    VT e[kRowsPerGroup];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      const bool ok = r < rows && tok[r] >= 0 && tok[r] < a.vocab;
      e[r] = ok ? *(const VT*)((const T*)a.E + (int64_t)tok[r] * a.d + N * c)
                : VT{};
    }
    // Encoding of coordinates N c .. N c + N - 1 (N / 2 sin/cos pairs):
    // frequency and angle in double precision, the angle reduced to
    // [-pi, pi] there (2 pi split in two parts, so the reduction adds less
    // than 1e-15 * |angle / 2 pi| of error), then a single-precision sine
    // and cosine of the reduced angle (error ~1e-7).
    FV pe;
#pragma unroll
    for (int q = 0; q < N / 2; ++q) {
      const int i = (N * c) / 2 + q;  // pair index
      const double w = exp2(-(2.0 * i / (double)a.d) * kLog2_10000);
      const double ang = pos * w;
      const double k = rint(ang * kInv2Pi);
      const double red = fma(-k, k2PiLo, fma(-k, k2PiHi, ang));
      float sf, cf;
      sincosf((float)red, &sf, &cf);
      pe[2 * q] = sf;
      pe[2 * q + 1] = cf;
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      if (r >= rows) break;
      const bool ok = tok[r] >= 0 && tok[r] < a.vocab;
      FV v;
#pragma unroll
      for (int k = 0; k < N; ++k) v[k] = ok ? (float)e[r][k] * scale + pe[k] : __builtin_nanf("");
      T* dst = (T*)a.out + ((int64_t)(b0 + r) * a.n + p) * a.d + N * c;
      if constexpr (N == 8) *(VT*)dst = __builtin_convertvector(v, VT);
      else *(VT*)dst = v;
    }
  }
}

template <typename T>
hipError_t launch_t(const EmbedArgs& a, hipStream_t s, LaunchEvents ev) {
  const int chunks = a.d / Vec<T>::N;
  const int threads = min(256, (chunks + 63) / 64 * 64);
  dim3 grid(a.n, (a.B + kRowsPerGroup - 1) / kRowsPerGroup);
  void* args[] = {(void*)&a};
  return launch_kernel((const void*)embed_positional_kernel<T>, grid, dim3(threads), args, 0,
                            s, ev.start, ev.stop, 0);
}

}  // namespace

hipError_t launch_embed_positional(const EmbedArgs& a, int f32, hipStream_t s, LaunchEvents ev) {
  if (a.B <= 0 || a.n <= 0 || a.d <= 0 || a.d % 8 != 0 ||
      (a.B + kRowsPerGroup - 1) / kRowsPerGroup > 65535)
    return hipErrorInvalidValue;
  return f32 ? launch_t<float>(a, s, ev) : launch_t<__bf16>(a, s, ev);
}

}  // namespace mha
