// prologue.hip -- per-head q/k RMSNorm followed by RoPE, one bf16 rounding.
//
// Work items of RL-Kernel issue #415 (Gemma-4-31B-it RFC, section 5):
// qk_rmsnorm_d256_d512, sliding_rope_d256 (standard RoPE, theta 1e4) and
// global_proportional_p_rope (partial 0.25, theta 1e6). Order and weight form as the
// TensorFold PR #1186 commit for tf_qk_rows_once states them: the weight multiplies the
// normalised row, and the rotation follows the norm.
//
// One work-group per token, one wave per head row. A lane holds D/64 consecutive
// values of the row; the sum of squares is a fixed per-lane sequential sum followed by
// a butterfly over the wave, so every lane ends with the same bits. The rotation
// partner of a value sits D/64-aligned in the lane `pair_offset / (D/64)` away.
// Angles are computed in fp64 (position * theta^(-2i/F)) once per token and pair,
// and their cos/sin rounded to fp32.
#include "launch.hpp"

namespace g4 {

template <int N>
struct alignas(2 * N) Bf16Vec {
  uint16_t v[N];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // hardware round to nearest even
}

template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(const PrologueArgs a) {
  constexpr int kPer = D / 64;
  __shared__ float cos_t[D / 2];
  __shared__ float sin_t[D / 2];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = a.rope_dims >> 1;
  const int pos = a.positions[t];
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv_freq = pow(a.rope_theta, -2.0 * (double)i / (double)a.rope_freq_dim);
    const double ang = (double)pos * inv_freq;
    double sv, cv;
    sincos(ang, &sv, &cv);
    cos_t[i] = (float)cv;
    sin_t[i] = (float)sv;
  }
  __syncthreads();

  const int64_t dst = a.kv_dst_row ? a.kv_dst_row[t] : t;
  const int nq = a.q_in ? a.num_q_heads : 0;
  const int nk = (a.k_in && dst >= 0) ? a.num_kv_heads : 0;
  const int nv = (a.v_in && dst >= 0) ? a.num_kv_heads : 0;
  const int d0 = lane * kPer;
  const int partner = a.pair_offset / kPer;  // lane distance between rotation partners
  const bool first_half = d0 < half;
  const bool second_half = d0 >= a.pair_offset && d0 < a.pair_offset + half;

  for (int r = wave; r < nq + nk + nv; r += 4) {
    const uint16_t* src;
    uint16_t* out;
    const uint16_t* w = nullptr;
    if (r < nq) {
      src = a.q_in + (t * a.num_q_heads + r) * D;
      out = a.q_out + (t * a.num_q_heads + r) * D;
      w = a.q_norm_w;
    } else if (r < nq + nk) {
      const int g = r - nq;
      src = a.k_in + (t * a.num_kv_heads + g) * D;
      out = a.k_out + (dst * a.num_kv_heads + g) * D;
      w = a.k_norm_w;
    } else {
      const int g = r - nq - nk;
      src = a.v_in + (t * a.num_kv_heads + g) * D;
      out = a.v_out + (dst * a.num_kv_heads + g) * D;
    }
    const Bf16Vec<kPer> xin = *reinterpret_cast<const Bf16Vec<kPer>*>(src + d0);
    if (w == nullptr) {  // raw V copy into the cache row
      *reinterpret_cast<Bf16Vec<kPer>*>(out + d0) = xin;
      continue;
    }
    const Bf16Vec<kPer> win = *reinterpret_cast<const Bf16Vec<kPer>*>(w + d0);
    float x[kPer];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      x[e] = bf16_to_f32(xin.v[e]);
      ss = ss + x[e] * x[e];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    const float inv_rms = 1.0f / sqrtf(ss * (1.0f / (float)D) + a.rms_eps);
    float y[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) y[e] = bf16_to_f32(win.v[e]) * (x[e] * inv_rms);
    if (half > 0) {
      float other[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) other[e] = __shfl_xor(y[e], partner);
      if (first_half) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int i = d0 + e;
          y[e] = y[e] * cos_t[i] - other[e] * sin_t[i];
        }
      } else if (second_half) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int i = d0 + e - a.pair_offset;
          y[e] = y[e] * cos_t[i] + other[e] * sin_t[i];
        }
      }
    }
    Bf16Vec<kPer> yo;
#pragma unroll
    for (int e = 0; e < kPer; ++e) yo.v[e] = f32_to_bf16(y[e]);
    *reinterpret_cast<Bf16Vec<kPer>*>(out + d0) = yo;
  }
}

hipError_t launch_prologue(int head_dim, const PrologueArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_tokens);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(prologue_kernel<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(prologue_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(prologue_kernel<256>, grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(prologue_kernel<512>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace g4
