// backward.hip -- deterministic gradients of the prefill attention for gfx950.
//
// The gradients of the attention with respect to q, k and v, for a trainer that runs the
// same declared arithmetic as the rollout's forward (RL-Kernel issue #415, Gemma-4-31B-it
// RFC, section 1; section 5, global_k_eq_v_projection: the one tensor that serves as K and
// V takes the gradient of both roles). With s = scale q k^T over the visible keys,
// P = softmax(s) and delta_i = dO_i . o_i (o the forward output the caller holds):
//   dS = P (dO v^T - delta),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T dO.
// No atomics and no split of any reduction: every gradient element is the accumulation of
// one work-group over 32-key blocks (dq) or 32-row tiles (dk, dv) in ascending order,
// aligned to position 0 of its sequence, so its bits do not depend on batch composition,
// packing or padding.
//
// Declared arithmetic: scores in fp32 (the forward's MFMA chain over the head dim);
// lse = m + log2(l), the row's log2 sum of exp2(s c) (c = scale log2 e) from an exact fp32
// running maximum and sum over the blocks in ascending order; P = exp2(fma(s, c, -lse));
// delta from fp32 products of the bf16 dO and out, summed in dim order then over the two
// lane halves; dS = P (dP - delta) in fp32; P and dS rounded to bf16 as the MFMA operands
// of dv, dk and dq; fp32 accumulation; the scale applied once to the dq and dk sums; one
// bf16 rounding of each output. For K = V one fp32 accumulator takes both roles at every
// step (dv's P^T dO, then dk's dS^T q), so the scale goes into dS before its bf16
// rounding: dk = bf16(sum of P^T dO + bf16(scale dS)^T q).
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace g4 {
namespace {

// Global -> LDS, 4 bytes per lane (lane i fills bytes 4 i .. 4 i + 3 of the 256 at `lds`).
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds" ::"s"(lds),
      "v"(voff), "s"(rsrc)
      : "memory");
}

// A 32-row tile of a bf16 tensor into LDS in the swizzled block layout of the forward's
// key blocks (tile.hpp): each wave issues kTileLoads 1 KiB loads. Row r of the tile starts
// row_off(r) bytes after `base`; rows at or past the record count read as zero.
template <int D>
constexpr int kTileLoads = Geom<D>::kBlockBytes / 1024 / kWaves;

template <int D, typename RowOff>
__device__ __forceinline__ void stage_tile(uint32_t lds, const void* base, uint32_t nrec, RowOff row_off, int wave,
                                           int lane) {
  constexpr int R = Geom<D>::kRowBytes;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc_uniform(base, nrec);
#pragma unroll
  for (int i = 0; i < kTileLoads<D>; ++i) {
    const int slot = wave + kWaves * i;
    const int byte = slot * 1024 + lane * 16;
    const int row = byte / R;
    const int chunk = ((byte % R) >> 4) ^ chunk_swizzle<D>(row);
    dma_b128(rs, __builtin_amdgcn_readfirstlane(lds + (uint32_t)(slot * 1024)), row_off(row) + (uint32_t)chunk * 16);
  }
}

// Wait until at most N of this wave's vector loads are in flight, then meet the waves
// (the counts name the loads issued after the awaited tile).
template <int N>
__device__ __forceinline__ void wait_tile() {
  wait_barrier<N>();
}

// bf16(x * scale) of 4 accumulator values.
__device__ __forceinline__ bf16x4_t scaled4(const f32x16_t& acc, int g4, float scale) {
  bf16x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[4 * g4 + e] * scale);
  return v;
}

// The forward's fragment reads from a tile stage at a compile-time extra byte offset (the
// second tile of a stage): a score-pattern read of k-step kk (32 rows x 16 dims) and a
// transpose-read pair of chunk c, key step k2 (32 dims x 16 rows).
template <int D, int EXTRA>
__device__ __forceinline__ u32x4_t k_read_at(const BlockAddr& ba, int kk) {
  const uint32_t a = ba.k[kk & 7];
  switch (kk >> 3) {
    case 0: return asm_read_b128_at<EXTRA>(a);
    case 1: return asm_read_b128_at<EXTRA + 256>(a);
    case 2: return asm_read_b128_at<EXTRA + 512>(a);
    default: return asm_read_b128_at<EXTRA + 768>(a);
  }
}

template <int D, int EXTRA>
__device__ __forceinline__ VPair v_read_at(const BlockAddr& ba, int c, int k2) {
  constexpr int R16 = 16 * Geom<D>::kRowBytes;
  const int c4 = c & 3;
  switch (((c >> 2) << 1) | k2) {
    case 0: return v_read_off<D, EXTRA>(ba, c4);
    case 1: return v_read_off<D, EXTRA + R16>(ba, c4);
    case 2: return v_read_off<D, EXTRA + 256>(ba, c4);
    case 3: return v_read_off<D, EXTRA + 256 + R16>(ba, c4);
    case 4: return v_read_off<D, EXTRA + 512>(ba, c4);
    case 5: return v_read_off<D, EXTRA + 512 + R16>(ba, c4);
    case 6: return v_read_off<D, EXTRA + 768>(ba, c4);
    default: return v_read_off<D, EXTRA + 768 + R16>(ba, c4);
  }
}

// Waits until at most N LDS operations are in flight; the fragments are named so no use
// of them moves above the wait.
template <int N>
__device__ __forceinline__ void lds_wait2(u32x4_t& a, u32x4_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait2(VPair& a, VPair& b) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a.lo), "+v"(a.hi), "+v"(b.lo), "+v"(b.hi) : "i"(N));
}

// Reads issued ahead of their MFMAs in the backward's pipelined tile steps.
constexpr int kBwdPf = 2;

}  // namespace

// ---------------------------------------------------------------------------------------
// dq and the row statistics. Work-group: 4 waves x 32 rows = 128 rows (positions x the G
// query heads of one KV head, position-major, as the forward's one-N-block form), over
// the same 32-key blocks as the forward, in ascending order. A first sweep over the blocks
// forms each row's lse; the next sweeps (one per part of the head dims: the 512-dim head
// keeps q, dO and half of dq in registers at a time) recompute P, dP and dS per block and
// accumulate dq^T += K^T dS^T with the forward's P*V instruction pattern (K read
// transposed from LDS). K and V blocks stream global -> LDS through NS stages (up to four,
// as the LDS allows), block j + NS - 1 issued as block j's work begins.
template <int D, bool KEQV>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(const BackwardArgs a) {
  constexpr int R = Geom<D>::kRowBytes;
  constexpr int KS = Geom<D>::kKSteps;
  constexpr int kTile = Geom<D>::kBlockBytes;
  constexpr int kStage = kTile * (KEQV ? 1 : 2);
  constexpr int kLoads = kTileLoads<D> * (KEQV ? 1 : 2);  // loads per wave per block
  constexpr int kPasses = D >= 512 ? 2 : 1;
  constexpr int NCH = Geom<D>::kDChunks / kPasses;  // 32-dim chunks of dq per sweep
  constexpr int NS = std::min(4, 160 * 1024 / kStage);  // stages
  static_assert(NS >= 2 && (NS - 1) * kLoads <= 63, "dq stages");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * kStage];
  lds_char_t* smem = lds_ptr(smem_raw);
  const uint32_t smem0 = lds_addr(smem);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int lgG = __builtin_ctz((unsigned)G);
  const int pairs = Hkv * a.batch;
  // (the last query blocks, which see the most keys, start first)
  const int pair = (int)(blockIdx.x % (unsigned)pairs);
  const int qb = a.num_qblocks - 1 - (int)(blockIdx.x / (unsigned)pairs);
  const int g = pair % Hkv;
  const int b = pair / Hkv;
  const int L = a.seq_len[b];
  const int s0 = a.seq_start[b];
  const int pos_per_group = kRowsPerGroup >> lgG;
  const int p0 = qb * pos_per_group;
  if (p0 >= L) return;
  const int rho = wave * kSlots + (lane & (kSlots - 1));
  const int qp = p0 + (rho >> lgG);
  const bool valid = qp < L;
  const int h = g * G + (rho & (G - 1));
  const RowBounds rb = row_bounds(valid ? qp : -1, a.window);
  const int64_t qrow = (int64_t)s0 + (valid ? qp : p0);
  const int64_t qoff = (qrow * Hq + h) * D;

  // The row's q and dO fragments (the B operands of S^T = K q^T and dP^T = V dO^T) and
  // delta = dO . out (this lane's dims in order, then the two lane halves).
  bf16x8_t qf[KS], dof[KS];
  load_q<D>(qf, a.q + qoff, valid, lane);
  load_q<D>(dof, a.dout + qoff, valid, lane);
  float dpart = 0.0f;
  {
    bf16x8_t of[KS];
    load_q<D>(of, a.out + qoff, valid, lane);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = dpart + (float)dof[kk][e] * (float)of[kk][e];
    }
  }
  const float delta = row_sum(dpart);
  // (a wait the compiler sees: its own loads are done before the block loads start)
  __builtin_amdgcn_s_waitcnt(VmCnt<0>::kImm);

  const int p_last = min(p0 + pos_per_group - 1, L - 1);
  const int jf = a.window > 0 ? max(0, p0 - a.window + 1) / kBlockKeys : 0;
  const int jl = p_last / kBlockKeys;
  const uint32_t stride = (uint32_t)Hkv * R;
  const int64_t head0 = ((int64_t)s0 * Hkv + g) * D;
  const char* kbase = reinterpret_cast<const char*>(a.k + head0);
  const char* vbase = reinterpret_cast<const char*>(a.v + head0);
  auto issue = [&](int j, int stage) {
    const int pos = j * kBlockKeys;
    const uint32_t nrec = (uint32_t)(min(L - pos, kBlockKeys) - 1) * stride + R;
    auto row_off = [&](int r) { return (uint32_t)r * stride; };
    stage_tile<D>(smem0 + (uint32_t)(stage * kStage), kbase + (int64_t)pos * stride, nrec, row_off, wave, lane);
    if constexpr (!KEQV)
      stage_tile<D>(smem0 + (uint32_t)(stage * kStage + kTile), vbase + (int64_t)pos * stride, nrec, row_off, wave,
                    lane);
  };
  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  const float c = a.scale_log2;
  // Wait for the block that has `newer` blocks issued after it, then meet the waves.
  auto wait_block = [&](int newer) {
    if (NS >= 4 && newer >= 3) {
      wait_tile<3 * kLoads>();
    } else if (NS >= 3 && newer == 2) {
      wait_tile<2 * kLoads>();
    } else if (newer == 1) {
      wait_tile<kLoads>();
    } else {
      wait_tile<0>();
    }
  };
  // The stage loop of a sweep over the blocks jf .. jl in ascending order: blocks jf ..
  // jf + NS - 2 ahead of the first, then at block j (stage stg) block j + NS - 1 into the
  // stage block j - 1 left; step(j, stg) runs the block, then the waves meet.
  auto stages = [&](auto step) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) {
      if (jf + t <= jl) issue(jf + t, t);
    }
    int stg = 0;
    for (int j = jf; j <= jl; ++j) {
      if (j + NS - 1 <= jl) issue(j + NS - 1, stg == 0 ? NS - 1 : stg - 1);
      wait_block(min(jl, j + NS - 1) - j);
      step(j, stg);
      lds_barrier();  // every wave is done with stage stg before it is loaded again
      stg = stg + 1 == NS ? 0 : stg + 1;
    }
    return stg;
  };
  // One sweep: body(j, K rows, V rows).
  auto sweep = [&](auto body) {
    stages([&](int j, int stg) {
      const lds_char_t* kst = smem + stg * kStage;
      body(j, kst, KEQV ? kst : kst + kTile);
    });
  };

  // Head dims up to 256 (q, dO and all of dq leave registers for reads in flight): the
  // stage is read through per-lane addresses that move with the stage, plus compile-time
  // offsets (the V tile's, the k-step's), kBwdPf steps ahead of the MFMAs, waiting on the
  // LDS counter; the same MFMA chains in the same order as the plain form below, so the
  // same bits.
  if constexpr (D <= 256) {
    static_assert(kPasses == 1, "one sweep of dq");
    BlockAddr ba;
    block_addr_init<D>(ba, lo, smem0, smem0, lane);
    constexpr int RING = kBwdPf + 1;
    constexpr int kVt = KEQV ? 0 : kTile;  // V rows after the K rows of a stage
    // S^T (K rows of the stage at OFF) and, with kDp, dP^T (its V rows): one read per
    // step for K = V (the fragment feeds both chains), two with separate V.
    auto chains = [&](auto off_c, auto dp_c, f32x16_t& s, f32x16_t& dp) {
      constexpr int OFF = decltype(off_c)::value;
      constexpr bool kDp = decltype(dp_c)::value;
      constexpr bool kTwo = kDp && !KEQV;
      constexpr int kReads = kTwo ? 2 : 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
      }
      u32x4_t ka[RING], va[RING];
#pragma unroll
      for (int q = 0; q < kBwdPf; ++q) {
        ka[q] = k_read_at<D, OFF>(ba, q);
        if constexpr (kTwo) va[q] = k_read_at<D, OFF + kVt>(ba, q);
      }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + kBwdPf < KS) {
          ka[(kk + kBwdPf) % RING] = k_read_at<D, OFF>(ba, kk + kBwdPf);
          if constexpr (kTwo) va[(kk + kBwdPf) % RING] = k_read_at<D, OFF + kVt>(ba, kk + kBwdPf);
        }
        const int after = kReads * ((kk + kBwdPf < KS ? kk + kBwdPf : KS - 1) - kk);
        u32x4_t& f = ka[kk % RING];
        u32x4_t& fv = va[kk % RING];
        if constexpr (kTwo) {
          if (after >= 4) {
            lds_wait2<4>(f, fv);
          } else if (after == 2) {
            lds_wait2<2>(f, fv);
          } else {
            lds_wait2<0>(f, fv);
          }
        } else {
          if (after >= 2) {
            lds_wait<2>(f);
          } else if (after == 1) {
            lds_wait<1>(f);
          } else {
            lds_wait<0>(f);
          }
        }
        s = mfma(as_bf16x8(f), qf[kk], s);
        if constexpr (kDp) dp = mfma(as_bf16x8(kTwo ? fv : f), dof[kk], dp);
      }
    };
    // (the fragment addresses follow the stage: moved after each block, back to stage 0
    // after the sweep)
    auto sweep_k = [&](auto body) {
      const int last = stages([&](int j, int stg) {
        body(j, std::integral_constant<int, 0>{});
        const int d = (stg + 1 == NS ? -(NS - 1) : 1) * kStage;
        block_addr_move(ba, d, d);
      });
      block_addr_move(ba, -last * kStage, -last * kStage);
    };
    // Sweep 1: lse (as below).
    float m = kNegInf, l = 0.0f;
    sweep_k([&](int j, auto off_c) {
      f32x16_t s, dp;
      chains(off_c, std::false_type{}, s, dp);
      mask_block(s, j * kBlockKeys + 4 * (lane >> 5), rb);
      const float mn = fmaxf(m, row_max(block_max(s)) * c);
      const float off = mn == kNegInf ? 0.0f : mn;
      const float alpha = mn == kNegInf ? 1.0f : exp2_hw(m - mn);
      float u = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) u = u + exp2_hw(__builtin_fmaf(s[r], c, -off));
      l = alpha * l + row_sum(u);
      m = mn;
    });
    const float lse = valid ? m + log2f(l) : 0.0f;
    if (valid && lane < kSlots) {
      a.lse[qrow * Hq + h] = lse;
      a.delta[qrow * Hq + h] = delta;
    }
    // Sweep 2: dq^T += K^T dS^T, the K^T transpose-read pairs kBwdPf steps ahead.
    f32x16_t acc[NCH];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cc][r] = 0.0f;
    }
    sweep_k([&](int j, auto off_c) {
      constexpr int OFF = decltype(off_c)::value;
      f32x16_t s, dp;
      chains(off_c, std::true_type{}, s, dp);
      mask_block(s, j * kBlockKeys + 4 * (lane >> 5), rb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(__builtin_fmaf(s[r], c, -lse));
        s[r] = p * (dp[r] - delta);
      }
      bf16x8_t df[2];
      pack_p(s, df);
      constexpr int T = 2 * NCH;
      VPair fv[RING];
#pragma unroll
      for (int q = 0; q < kBwdPf; ++q) fv[q] = v_read_at<D, OFF>(ba, q / 2, q & 1);
#pragma unroll
      for (int i = 0; i < T; ++i) {
        if (i + kBwdPf < T) {
          const int n = i + kBwdPf;
          fv[n % RING] = v_read_at<D, OFF>(ba, n / 2, n & 1);
        }
        const int after = 2 * ((i + kBwdPf < T ? i + kBwdPf : T - 1) - i);
        VPair& f = fv[i % RING];
        if (after >= 4) {
          lds_wait<4>(f);
        } else if (after == 2) {
          lds_wait<2>(f);
        } else {
          lds_wait<0>(f);
        }
        acc[i / 2] = mfma(as_bf16x8(f), df[i & 1], acc[i / 2]);
      }
    });
    if (valid) {
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          *reinterpret_cast<bf16x4_t*>(a.dq + qoff + 32 * cc + 8 * g4 + 4 * (lane >> 5)) = scaled4(acc[cc], g4, a.scale);
        }
      }
    }
    return;
  }

  // Sweep 1: lse, from an exact running maximum and sum (log2 units).
  float m = kNegInf, l = 0.0f;
  sweep([&](int j, const lds_char_t* kst, const lds_char_t*) {
    f32x16_t s = score_block<D>(kst, lo, qf);
    mask_block(s, j * kBlockKeys + 4 * (lane >> 5), rb);
    const float mn = fmaxf(m, row_max(block_max(s)) * c);
    const float off = mn == kNegInf ? 0.0f : mn;
    const float alpha = mn == kNegInf ? 1.0f : exp2_hw(m - mn);
    float u = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) u = u + exp2_hw(__builtin_fmaf(s[r], c, -off));
    l = alpha * l + row_sum(u);
    m = mn;
  });
  const float lse = valid ? m + log2f(l) : 0.0f;
  if (valid && lane < kSlots) {
    a.lse[qrow * Hq + h] = lse;
    a.delta[qrow * Hq + h] = delta;
  }

  // Sweeps 2 ..: dq^T for NCH chunks of the head dims at a time.
  for (int pass = 0; pass < kPasses; ++pass) {
    f32x16_t acc[NCH];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cc][r] = 0.0f;
    }
    sweep([&](int j, const lds_char_t* kst, const lds_char_t* vst) {
      f32x16_t s = score_block<D>(kst, lo, qf);
      mask_block(s, j * kBlockKeys + 4 * (lane >> 5), rb);
      const f32x16_t dp = score_block<D>(vst, lo, dof);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(__builtin_fmaf(s[r], c, -lse));
        s[r] = p * (dp[r] - delta);
      }
      bf16x8_t df[2];
      pack_p(s, df);
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        acc[cc] = mfma(v_fragment<D>(kst, lo, pass * NCH + cc, 0), df[0], acc[cc]);
        acc[cc] = mfma(v_fragment<D>(kst, lo, pass * NCH + cc, 1), df[1], acc[cc]);
      }
    });
    if (valid) {
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          *reinterpret_cast<bf16x4_t*>(a.dq + qoff + 32 * (pass * NCH + cc) + 8 * g4 + 4 * (lane >> 5)) =
              scaled4(acc[cc], g4, a.scale);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// dk and dv. Work-group: 4 waves x 32 keys = 128 consecutive keys of one (sequence, KV
// head); wave w owns keys K0 + 32 w .. + 31 (its k and v fragments stay in registers as
// the B operands of S = q K^T and dP = dO V^T). The rows that can see the work-group's
// keys come in 32-row tiles (positions x the G query heads, position-major; tiles start at
// row 0 of the sequence) in ascending order, global -> LDS in two stages with their lse
// and delta. Per tile: S and dP with lane = key and registers = rows (the forward's score
// pattern with the roles of the LDS rows and the register fragments exchanged), P and dS,
// then dv^T += dO^T P and dk^T += q^T dS with the forward's P*V pattern (dO and q read
// transposed from LDS). Rows that do not see a key add exact zeros to it. The head dims
// go in parts where the accumulators would not fit the register file, one work-group per
// part (each recomputes S and dP): the parts of the heaviest key blocks run side by side
// rather than one after the other.
template <int D, bool KEQV>
constexpr int dkv_parts() { return D >= 512 ? (KEQV ? 2 : 4) : 1; }

template <int D, bool KEQV>
__global__ __launch_bounds__(kThreads, 1) void dkv_kernel(const BackwardArgs a) {
  constexpr int R = Geom<D>::kRowBytes;
  constexpr int KS = Geom<D>::kKSteps;
  constexpr int kTile = Geom<D>::kBlockBytes;
  constexpr int kStage = 2 * kTile + 512;  // q rows, dO rows, lse (256 B), delta (256 B)
  constexpr int kLoads = 2 * kTileLoads<D> + 2;  // loads per wave per tile
  constexpr int kPasses = dkv_parts<D, KEQV>();
  constexpr int NCH = Geom<D>::kDChunks / kPasses;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kStage];
  lds_char_t* smem = lds_ptr(smem_raw);
  const uint32_t smem0 = lds_addr(smem);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int lgG = __builtin_ctz((unsigned)G);
  const int pairs = Hkv * a.batch;
  // (key block slowest: the heaviest blocks, those of the first keys, start first)
  const int pair = (int)(blockIdx.x % (unsigned)pairs);
  const int pass = (int)((blockIdx.x / (unsigned)pairs) % (unsigned)kPasses);
  const int kb = (int)(blockIdx.x / (unsigned)(pairs * kPasses));
  const int g = pair % Hkv;
  const int b = pair / Hkv;
  const int L = a.seq_len[b];
  const int s0 = a.seq_start[b];
  const int K0 = kb * kRowsPerGroup;
  if (K0 >= L) return;
  const int key = K0 + wave * kSlots + (lane & (kSlots - 1));
  const bool kvalid = key < L;
  const int64_t krow = (int64_t)s0 + (kvalid ? key : K0);
  const int64_t koff = (krow * Hkv + g) * D;
  bf16x8_t kf[KS], vf[KS];
  load_q<D>(kf, a.k + koff, kvalid, lane);
  if constexpr (!KEQV) load_q<D>(vf, a.v + koff, kvalid, lane);
  __builtin_amdgcn_s_waitcnt(VmCnt<0>::kImm);

  // Tiles of rows that see keys K0 .. K0 + 127: from the row of position K0 to the last
  // row of the last position that sees one of them.
  const int pos_last = a.window > 0 ? min(L - 1, K0 + kRowsPerGroup - 1 + a.window - 1) : L - 1;
  const int t0 = (K0 << lgG) / kSlots;
  const int t1 = (((pos_last + 1) << lgG) - 1) / kSlots;
  const int tile_pos = kSlots >> lgG;  // positions per tile
  const uint32_t qstride = (uint32_t)Hq * R;
  auto issue = [&](int t, int stage) {
    const int pt0 = t * tile_pos;
    const int npos = min(L - pt0, tile_pos);
    const int64_t row0 = ((int64_t)(s0 + pt0) * Hq + g * G);
    const uint32_t nrec = (uint32_t)(npos - 1) * qstride + (uint32_t)G * R;
    auto row_off = [&](int r) { return (uint32_t)(r >> lgG) * qstride + (uint32_t)(r & (G - 1)) * R; };
    const uint32_t st = smem0 + (uint32_t)(stage * kStage);
    stage_tile<D>(st, a.q + row0 * D, nrec, row_off, wave, lane);
    stage_tile<D>(st + kTile, a.dout + row0 * D, nrec, row_off, wave, lane);
    // lse and delta of the tile's 32 rows (lanes 32 .. 63 read past the records: zero)
    const uint32_t snrec = (uint32_t)((npos - 1) * Hq + G) * 4;
    const uint32_t soff =
        lane < kSlots ? (uint32_t)(((lane >> lgG) * Hq + (lane & (G - 1))) * 4) : kOutOfRange;
    dma_b32(make_rsrc_uniform(a.lse + row0, snrec), __builtin_amdgcn_readfirstlane(st + 2 * kTile), soff);
    dma_b32(make_rsrc_uniform(a.delta + row0, snrec), __builtin_amdgcn_readfirstlane(st + 2 * kTile + 256), soff);
  };
  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  const float c = a.scale_log2;
  const int kbase = 4 * (lane >> 5);  // this lane's first row of each 8-row group
  // fragment addresses of stage 0 (moved to the other stage tile by tile); the
  // transpose reads start at this part's dims (NCH / 4 groups of 256 bytes per part), so
  // the chunk index within a read is a compile-time value
  static_assert(kPasses == 1 || NCH % 4 == 0, "a part covers whole 4-chunk groups");
  BlockAddr ba;
  block_addr_init<D>(ba, lo, smem0, smem0, lane);
  block_addr_move(ba, 0, pass * 256 * (NCH / 4));

  {
    // (one tensor as K and V: one accumulator takes both roles, dv's P^T dO and dk's
    // (scale dS)^T q, in that order at every step)
    constexpr int NDV = KEQV ? 1 : NCH;
    f32x16_t dk_acc[NCH], dv_acc[NDV];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk_acc[cc][r] = 0.0f;
        if constexpr (!KEQV) dv_acc[cc][r] = 0.0f;
      }
    }
    issue(t0, 0);
    for (int t = t0; t <= t1; ++t) {
      const int stg = (t - t0) & 1;
      if (t < t1) {
        issue(t + 1, stg ^ 1);
        wait_tile<kLoads>();
      } else {
        wait_tile<0>();
      }
      const lds_char_t* qst = smem + stg * kStage;
      const lds_f32_t* lse_s = reinterpret_cast<const lds_f32_t*>(qst + 2 * kTile);
      const lds_f32_t* del_s = reinterpret_cast<const lds_f32_t*>(qst + 2 * kTile + 256);
      // S^T and dP^T (lane = key): two MFMA chains over the head dims, the q rows and the
      // dO rows of the stage read kBwdPf k-steps ahead (two reads per step).
      f32x16_t s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
      }
      {
        constexpr int RING = kBwdPf + 1;
        u32x4_t qa[RING], da[RING];
#pragma unroll
        for (int q = 0; q < kBwdPf; ++q) {
          qa[q] = k_read_at<D, 0>(ba, q);
          da[q] = k_read_at<D, kTile>(ba, q);
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          if (kk + kBwdPf < KS) {
            qa[(kk + kBwdPf) % RING] = k_read_at<D, 0>(ba, kk + kBwdPf);
            da[(kk + kBwdPf) % RING] = k_read_at<D, kTile>(ba, kk + kBwdPf);
          }
          const int after = 2 * ((kk + kBwdPf < KS ? kk + kBwdPf : KS - 1) - kk);
          u32x4_t& fq = qa[kk % RING];
          u32x4_t& fd = da[kk % RING];
          if (after >= 4) {
            lds_wait2<4>(fq, fd);
          } else if (after == 2) {
            lds_wait2<2>(fq, fd);
          } else {
            lds_wait2<0>(fq, fd);
          }
          s = mfma(as_bf16x8(fq), kf[kk], s);
          dp = mfma(as_bf16x8(fd), KEQV ? kf[kk] : vf[kk], dp);
        }
      }
      // P and dS (rows that do not see the key: an argument of -inf, p = 0)
      const int pt0 = t * tile_pos;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + kbase + (r & 3);  // tile row of register r
        const int qpos = pt0 + (row >> lgG);
        const bool vis = kvalid && qpos < L && key <= qpos && (a.window == 0 || qpos - key < a.window);
        const float x = __builtin_fmaf(s[r], c, -lse_s[row]);
        const float p = exp2_hw(vis ? x : kNegInf);
        s[r] = p;
        if constexpr (KEQV) {
          dp[r] = p * (dp[r] - del_s[row]) * a.scale;
        } else {
          dp[r] = p * (dp[r] - del_s[row]);
        }
      }
      bf16x8_t pf[2], df[2];
      pack_p(s, pf);
      pack_p(dp, df);
      // dv^T += dO^T P and dk^T += q^T dS: per step one chunk and key step, the dO^T and
      // q^T transpose-read pairs read kBwdPf steps ahead (four reads per step).
      {
        constexpr int RING = kBwdPf + 1;
        constexpr int T = 2 * NCH;
        VPair fv[RING], fk[RING];
#pragma unroll
        for (int q = 0; q < kBwdPf; ++q) {
          fv[q] = v_read_at<D, kTile>(ba, q / 2, q & 1);
          fk[q] = v_read_at<D, 0>(ba, q / 2, q & 1);
        }
#pragma unroll
        for (int i = 0; i < T; ++i) {
          if (i + kBwdPf < T) {
            const int n = i + kBwdPf;
            fv[n % RING] = v_read_at<D, kTile>(ba, n / 2, n & 1);
            fk[n % RING] = v_read_at<D, 0>(ba, n / 2, n & 1);
          }
          const int after = 4 * ((i + kBwdPf < T ? i + kBwdPf : T - 1) - i);
          VPair& gv = fv[i % RING];
          VPair& gk = fk[i % RING];
          if (after >= 8) {
            lds_wait2<8>(gv, gk);
          } else if (after == 4) {
            lds_wait2<4>(gv, gk);
          } else {
            lds_wait2<0>(gv, gk);
          }
          if constexpr (KEQV) {
            dk_acc[i / 2] = mfma(as_bf16x8(gv), pf[i & 1], dk_acc[i / 2]);
          } else {
            dv_acc[i / 2] = mfma(as_bf16x8(gv), pf[i & 1], dv_acc[i / 2]);
          }
          dk_acc[i / 2] = mfma(as_bf16x8(gk), df[i & 1], dk_acc[i / 2]);
        }
      }
      // the next tile's stage
      block_addr_move(ba, stg ? -kStage : kStage, stg ? -kStage : kStage);
      lds_barrier();  // every wave is done with stage stg before it is loaded again
    }
    if (kvalid) {
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int64_t d0 = 32 * (pass * NCH + cc) + 8 * g4 + 4 * (lane >> 5);
          if constexpr (KEQV) {
            *reinterpret_cast<bf16x4_t*>(a.dk + koff + d0) = scaled4(dk_acc[cc], g4, 1.0f);
          } else {
            *reinterpret_cast<bf16x4_t*>(a.dk + koff + d0) = scaled4(dk_acc[cc], g4, a.scale);
            *reinterpret_cast<bf16x4_t*>(a.dv + koff + d0) = scaled4(dv_acc[cc], g4, 1.0f);
          }
        }
      }
    }
  }
}

template <int D, bool KEQV>
static hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t stream) {
  const unsigned pairs = (unsigned)(a.num_kv_heads * a.batch);
  hipLaunchKernelGGL((dq_kernel<D, KEQV>), dim3((unsigned)a.num_qblocks * pairs), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkv_kernel<D, KEQV>), dim3((unsigned)a.num_kblocks * pairs * (unsigned)dkv_parts<D, KEQV>()),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward(int head_dim, bool k_eq_v, const BackwardArgs& a, hipStream_t stream) {
#define G4_BACKWARD(DD)                                                         \
  if (head_dim == DD) {                                                         \
    return k_eq_v ? launch_backward_t<DD, true>(a, stream) : launch_backward_t<DD, false>(a, stream); \
  }
  G4_BACKWARD(64)
  G4_BACKWARD(128)
  G4_BACKWARD(256)
  G4_BACKWARD(512)
#undef G4_BACKWARD
  return hipErrorInvalidValue;
}

}  // namespace g4
