// prologue.hip -- per-head q/k RMSNorm followed by RoPE, one bf16 rounding.
//
// Work items of RL-Kernel issue #415 (Gemma-4-31B-it RFC, section 5):
// qk_rmsnorm_d256_d512, sliding_rope_d256 (standard RoPE, theta 1e4) and
// global_proportional_p_rope (partial 0.25, theta 1e6). Order and weight form as the
// TensorFold PR #1186 commit for tf_qk_rows_once states them: the weight multiplies the
// normalised row, and the rotation follows the norm.
#include "launch.hpp"

namespace g4 {

// Value e (0..7) of 8 packed bf16, as fp32. (Whole-word operations: an array of 16-bit
// elements indexed after a select ends up in scratch memory.)
__device__ __forceinline__ float bf16_at(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);  // hardware round to nearest even
}

__device__ __forceinline__ uint4 pack_bf16(const float (&y)[8]) {
  uint4 r;
  r.x = f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16);
  r.y = f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16);
  r.z = f32_to_bf16(y[4]) | (f32_to_bf16(y[5]) << 16);
  r.w = f32_to_bf16(y[6]) | (f32_to_bf16(y[7]) << 16);
  return r;
}

// Lane exchanges in registers (DPP moves and the gfx950 row swaps), not through the LDS
// unit as a general shuffle is: value of lane l ^ m within a 16-lane row for the masks
// the DPP controls give directly (quad permutations 1, 2, 3; half-row mirror 7; row
// mirror 15; row rotation by 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kXor3 = 0x1B, kXor7 = 0x141, kXor15 = 0x140, kXor8 = 0x128;

// The 16-lane row pair (or 32-lane half pair) swap leaves {x of the even row, x of the odd
// row} in (r[0], r[1]) in both rows.
__device__ __forceinline__ void swap16(float x, float& even, float& odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  even = __uint_as_float(r[0]);
  odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Sum over a row's kLanes consecutive lanes by a butterfly of lane-xor steps (masks 1, 3,
// 7, 15, then the 16- and 32-lane swaps): each step adds the same two values in both
// lanes of a pair, so every lane of the row ends with the same bits.
template <int kLanes>
__device__ __forceinline__ float row_lanes_sum(float s) {
  static_assert(kLanes >= 8 && kLanes <= 64, "lanes per row");
  s = s + dpp<kXor1>(s);
  s = s + dpp<kXor3>(s);
  s = s + dpp<kXor7>(s);
  if constexpr (kLanes >= 16) s = s + dpp<kXor15>(s);
  if constexpr (kLanes >= 32) {
    float a, b;
    swap16(s, a, b);
    s = a + b;
  }
  if constexpr (kLanes >= 64) {
    float a, b;
    swap32(s, a, b);
    s = a + b;
  }
  return s;
}

// other[e] = y[e] of lane l ^ m (m = the rotation partner's lane distance, a power of two).
__device__ __forceinline__ void lane_xor(float (&other)[8], const float (&y)[8], int m, int lane) {
  switch (m) {
    case 1:
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = dpp<kXor1>(y[e]);
      break;
    case 2:
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = dpp<kXor2>(y[e]);
      break;
    case 4:
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = dpp<kXor7>(dpp<kXor3>(y[e]));
      break;
    case 8:
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = dpp<kXor8>(y[e]);
      break;
    case 16: {
      const bool odd = (lane >> 4) & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float ev, od;
        swap16(y[e], ev, od);
        other[e] = odd ? ev : od;
      }
      break;
    }
    case 32: {
      const bool high = lane >= 32;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float lo, hi;
        swap32(y[e], lo, hi);
        other[e] = high ? lo : hi;
      }
      break;
    }
    default:
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = __shfl_xor(y[e], m);
  }
}

// One work-group per token, four waves. A head row of D values is held by D/8 lanes,
// 8 consecutive values (16 bytes) each, so one wave-wide load covers 512/D rows. The
// token's rows are numbered q heads, then k heads, then the raw v copies; wave w takes
// the row groups w, w + 4, ..., and issues all their loads (up to kBatch per wave at
// a time) before building the angle table, so the table's fp64 work runs while the
// reads are in flight. Many small work-groups per CU keep HBM busy: at least four
// per CU fit (the register budget that sets), and nine 16-byte loads per lane cover
// a 31B token (48 rows of 256 or 36 of 512 dims).
// The sum of squares is a fixed per-lane sequential sum of 8 squares followed by a
// butterfly over the row's lanes (row_lanes_sum), so every lane of a row ends with the
// same bits. The rotation partner of a value sits pair_offset / 8 lanes away in the same
// row (lane_xor).
// Angles: rope_cos_sin (launch.hpp), one table per token.
template <int D>
__global__ __launch_bounds__(256, 4) void prologue_kernel(const PrologueArgs a) {
  constexpr int kE = 8;                 // values per lane
  constexpr int kLanes = D / kE;        // lanes per row
  constexpr int kRowsPerLoad = 64 / kLanes;
  constexpr int kBatch = 9;             // row groups per wave held in registers at once
  __shared__ float cos_t[D / 2];
  __shared__ float sin_t[D / 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t = blockIdx.x;
  const int half = a.rope_dims >> 1;

  // Scalars and the norm weights first: global loads complete in order, so anything
  // read after the row loads would wait for them.
  const int pos = a.positions[t];
  const int64_t dst = a.kv_dst_row ? a.kv_dst_row[t] : t;
  const int nq = a.q_in ? a.num_q_heads : 0;
  const int nk = (a.k_in && dst >= 0) ? a.num_kv_heads : 0;
  const int nv = (a.v_in && dst >= 0) ? a.num_kv_heads : 0;
  const int rows = nq + nk + nv;
  const int groups = (rows + kRowsPerLoad - 1) / kRowsPerLoad;
  const int sub = lane / kLanes;        // row of this lane inside a load
  const int d0 = (lane % kLanes) * kE;  // first of this lane's 8 dims
  const int partner = a.pair_offset / kE;
  const bool first_half = d0 < half;
  const bool second_half = d0 >= a.pair_offset && d0 < a.pair_offset + half;
  const uint4 wq = a.q_in ? *reinterpret_cast<const uint4*>(a.q_norm_w + d0) : uint4{};
  const uint4 wk = a.k_in ? *reinterpret_cast<const uint4*>(a.k_norm_w + d0) : uint4{};

  // Row r of the token: kind (0 q, 1 k, 2 v), its source and destination rows.
  auto src_of = [&](int r) -> const uint16_t* {
    if (r < nq) return a.q_in + (t * a.num_q_heads + r) * D;
    if (r < nq + nk) return a.k_in + (t * a.num_kv_heads + (r - nq)) * D;
    return a.v_in + (t * a.num_kv_heads + (r - nq - nk)) * D;
  };
  auto dst_of = [&](int r) -> uint16_t* {
    if (r < nq) return a.q_out + (t * a.num_q_heads + r) * D;
    if (r < nq + nk) return a.k_out + (dst * a.num_kv_heads + (r - nq)) * D;
    return a.v_out + (dst * a.num_kv_heads + (r - nq - nk)) * D;
  };
  uint4 xin[kBatch];
  auto issue = [&](int base) {
#pragma unroll
    for (int it = 0; it < kBatch; ++it) {
      const int r = (base + wave + 4 * it) * kRowsPerLoad + sub;
      xin[it] = uint4{};
      if (r < rows) xin[it] = *reinterpret_cast<const uint4*>(src_of(r) + d0);
    }
  };
  issue(0);

  for (int i = tid; i < half; i += 256) {
    float cv, sv;
    rope_cos_sin(pos, i, a.rope_theta, a.rope_freq_dim, cv, sv);
    cos_t[i] = cv;
    sin_t[i] = sv;
  }
  __syncthreads();

  for (int base = 0; base < groups; base += 4 * kBatch) {
    if (base > 0) issue(base);
#pragma unroll
    for (int it = 0; it < kBatch; ++it) {
      if (base + 4 * it >= groups) break;  // uniform over the work-group
      const int r = (base + wave + 4 * it) * kRowsPerLoad + sub;
      const int kind = r < nq ? 0 : r < nq + nk ? 1 : 2;
      const uint4 wv = kind == 0 ? wq : wk;
      // Every lane runs the arithmetic (the shuffles need the whole wave); rows past
      // the token's last one store nothing, raw v copies store their input.
      float x8[kE];
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        x8[e] = bf16_at(xin[it], e);
        ss = ss + x8[e] * x8[e];
      }
      ss = row_lanes_sum<kLanes>(ss);
      const float inv_rms = 1.0f / sqrtf(ss * (1.0f / (float)D) + a.rms_eps);
      float xn[kE];  // the unit RMS norm of the row (a value row's result when v is normed)
      float y[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        xn[e] = x8[e] * inv_rms;
        y[e] = bf16_at(wv, e) * xn[e];
      }
      if (half > 0) {
        float other[kE];
        lane_xor(other, y, partner, lane);
        if (first_half) {
#pragma unroll
          for (int e = 0; e < kE; ++e) y[e] = y[e] * cos_t[d0 + e] - other[e] * sin_t[d0 + e];
        } else if (second_half) {
#pragma unroll
          for (int e = 0; e < kE; ++e) {
            const int i = d0 + e - a.pair_offset;
            y[e] = y[e] * cos_t[i] + other[e] * sin_t[i];
          }
        }
      }
      if (r < rows) {
        const uint4 val = kind != 2 ? pack_bf16(y) : a.v_norm ? pack_bf16(xn) : xin[it];
        *reinterpret_cast<uint4*>(dst_of(r) + d0) = val;
      }
    }
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
