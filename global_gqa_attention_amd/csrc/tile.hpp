// tile.hpp -- the per-block update of one wave's 32 query rows, shared by the prefill
// and decode kernels.
//
// What it computes follows the attention work items of RL-Kernel issue #415
// (Gemma-4-31B-it RFC, section 5: sliding_attention_core, global_attention_core) under
// that page's section 4 numerical contract: fp32 accumulation and one fixed order of
// every reduction of a row, whichever other rows share the work-group.
//
// Layout (gfx950, wave64):
//   * A wave owns 32 query slots (MFMA N). Keys come in blocks of 32 (MFMA M), aligned
//     to position 0 of the sequence and taken in ascending order. A block's scores are
//     computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16
//     dims read from LDS, B = the Q^T fragment held in registers, one accumulator chain
//     over the head dim in ascending 16-dim steps. Lane l then holds query slot l % 32
//     and 16 keys of the block: key(r) = 8 (r / 4) + 4 (l / 32) + (r % 4).
//   * The online softmax advances once per block. A slot's statistics live in lanes l
//     and l ^ 32; v_permlane32_swap finishes each row reduction.
//   * O^T = V^T P^T with the same instruction: A = 32 head dims x 16 keys read from LDS
//     with the gfx950 transpose read (ds_read_b64_tr_b16), B = P^T straight from the
//     score registers (rounded to bf16), two 16-key steps per block.
//   * LDS rows hold one key (D bf16) with 16-byte chunks XOR-swizzled by the key, which
//     keeps the score reads (16 lanes = 16 keys, one chunk) and the transpose reads
//     (4 keys x 4 chunks per 16 lanes) free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) float lds_f32_t;

// The LDS address of a __shared__ object.
template <typename T>
__device__ __forceinline__ lds_char_t* lds_ptr(T* p) {
  return (lds_char_t*)(p);
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char_t* p) { return (uint32_t)(uintptr_t)p; }

constexpr int kWave = 64;
constexpr int kSlots = 32;      // query slots per wave (MFMA N)
constexpr int kBlockKeys = 32;  // keys per block (MFMA M; unit of the softmax update)
constexpr int kWaves = 4;       // waves per work-group
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerGroup = kSlots * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A row's two lanes are l and l ^ 32. permlane32_swap leaves the pair {x_l, x_(l^32)}
// in (a, b) in every lane (lanes < 32 and >= 32 see the same two values in the same
// registers), so max(a, b) and a + b are the same bits in both lanes of the row.
__device__ __forceinline__ void row_pair(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float row_max(float x) {
  float a, b;
  row_pair(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float row_sum(float x) {
  float a, b;
  row_pair(x, a, b);
  return a + b;
}

template <int D>
struct Geom {
  static_assert(D == 64 || D == 128 || D == 256 || D == 512, "head dim");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKSteps = D / 16;            // score k-steps over the head dim
  static constexpr int kDChunks = D / 32;           // 32-dim output chunks
  static constexpr int kBlockBytes = kBlockKeys * kRowBytes;  // one block of K (or V)
};

// Physical 16-byte chunk of logical chunk c in key row `key`: c ^ swizzle(key).
template <int D>
__device__ __forceinline__ int chunk_swizzle(int key) {
  if constexpr (D >= 128) {
    return ((key & 3) << 2) | ((key >> 2) & 3);
  } else {
    return (key >> 1) & 7;
  }
}

// Per-wave running state of 32 query slots (lane l serves slot l % 32) for DO output
// dims.
template <int DO>
struct RowState {
  f32x16_t o[DO / 32];  // O^T chunk c: dim 32c + 8(r/4) + 4(l/32) + r%4
  float m;              // exponent offset (lazily updated running max, log2 units)
  float l;              // running sum of exp2(score - m)
};

template <int DO>
__device__ __forceinline__ void row_state_init(RowState<DO>& st) {
#pragma unroll
  for (int c = 0; c < DO / 32; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[c][r] = 0.0f;
  }
  st.m = kNegInf;
  st.l = 0.0f;
}

// Q^T fragments of this lane's slot: dims 16 kk + 8 (l/32) + 0..7.
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[Geom<D>::kKSteps], const uint16_t* qrow, bool valid, int lane) {
  const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(qrow + 8 * (lane >> 5));
#pragma unroll
  for (int kk = 0; kk < Geom<D>::kKSteps; ++kk) {
    if (valid) {
      qf[kk] = src[2 * kk];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
    }
  }
}

// Per-lane LDS byte offsets inside a block. The swizzle only touches the low four bits
// of a chunk index and depends only on the low four bits of the key, so every read of
// a block is one of 16 per-lane bases plus a compile-time offset.
template <int D>
struct LaneOffsets {
  uint32_t k[8];  // score reads: key (l % 32), chunk 2 kk + (l / 32), for kk % 8
  uint32_t v[8];  // transpose reads: [part * 4 + c % 4]
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  LaneOffsets<D> lo;
  const int key = lane & 31;
  const int sw = chunk_swizzle<D>(key);
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) {
    const int c = 2 * k8 + (lane >> 5);
    lo.k[k8] = (uint32_t)(key * Geom<D>::kRowBytes + ((c ^ sw) << 4));
  }
  const int grp = lane >> 4;
  const int e = 2 * (grp & 1) + ((lane & 3) >> 1);  // chunk within a 4-chunk (32-dim) group
  const int half = lane & 1;                        // 8-byte half of the chunk
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const int vkey = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * part;
    const int vsw = chunk_swizzle<D>(vkey);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      lo.v[part * 4 + c4] = (uint32_t)(vkey * Geom<D>::kRowBytes + (((4 * c4 + e) ^ vsw) << 4) + (half << 3));
    }
  }
  return lo;
}

// ---- S^T = K Q^T for one block ---------------------------------------------------
// One accumulator chain over the head dim, 16 dims per step, ascending; the K block's
// rows start at `kst`.
template <int D>
__device__ __forceinline__ f32x16_t score_block(const lds_char_t* kst, const LaneOffsets<D>& lo,
                                                const bf16x8_t (&qf)[Geom<D>::kKSteps]) {
  f32x16_t s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
  for (int kk = 0; kk < Geom<D>::kKSteps; ++kk) {
    const bf16x8_t a = *reinterpret_cast<const lds_bf16x8_t*>(kst + lo.k[kk & 7] + (kk >> 3) * 256);
    s = mfma(a, qf[kk], s);
  }
  return s;
}

// Visible key range of this lane's query row: keys lo..hi (hi < 0: no key).
struct RowBounds {
  int lo;
  int hi;
};

__device__ __forceinline__ RowBounds row_bounds(int qpos, int window) {
  RowBounds rb;
  rb.hi = qpos;
  rb.lo = (window > 0) ? qpos - window + 1 : -0x40000000;
  return rb;
}

// Hide the keys of a block outside the row's range (score -> -inf). The key of
// register r is key_pos0 + 8 (r/4) + (r%4), key_pos0 = block start + 4 (l/32). A row
// without keys (hi < 0) has hi - lo below every key - lo, so it hides everything.
__device__ __forceinline__ void mask_block(f32x16_t& s, int key_pos0, RowBounds rb) {
  const uint32_t span = (uint32_t)(rb.hi - rb.lo);  // visible iff (key - lo) <= span (unsigned)
  const int base = key_pos0 - rb.lo;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + (r & 3);
    s[r] = ((uint32_t)(base + off) <= span) ? s[r] : kNegInf;
  }
}

// Largest of this lane's 16 raw scores.
__device__ __forceinline__ float block_max(const f32x16_t& s) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  return mx;
}

// Threshold of the lazy max update, in log2 units: the exponent offset of a row only
// moves when a block's largest score exceeds it by more than this. Every probability is
// formed under the row's final offset (the kernels run a second pass from the final
// offsets when a row moved after holding keys), so probabilities stay <= 2^64 before
// normalisation, and l <= L 2^64 and |O| <= L 2^64 max|v| stay far inside fp32 for any
// finite bf16 V with L * max|v| < 2^63. A move needs a row's scores to span more than
// 64 / log2(e) ~ 44 natural units, which normalised queries and keys do not.
constexpr float kRescaleThreshold = 64.0f;

// A row's exponent offset for this block. m_old is the offset in use (-inf before the
// first visible key). Returns whether it moves; m_new is the new offset, alpha the
// factor of the old (l, O) (exactly 1 when the offset stays; 0 when the row held no key),
// `offset` the value subtracted from the scores (0 while the row has seen no visible key,
// so hidden keys give exp2(-inf) = 0). A block without visible keys leaves (m, l, O)
// unchanged. A move after the row held keys is reported to the caller, whose second pass
// starts from the final offset (there alpha is always 1).
__device__ __forceinline__ bool softmax_step(float m_old, float tile_max, float& m_new, float& alpha, float& offset) {
  const bool move = tile_max > m_old + kRescaleThreshold;
  m_new = move ? tile_max : m_old;
  alpha = move ? exp2_hw(m_old - m_new) : 1.0f;
  offset = (m_new == kNegInf) ? 0.0f : m_new;
  return move;
}

// p = exp2(s * c - offset) in place, one fused multiply-add (a single rounding) then
// the hardware exp2; returns this lane's sum of the 16 values in register order.
__device__ __forceinline__ float exp_block(f32x16_t& s, float scale_log2, float offset) {
  float u = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = exp2_hw(__builtin_fmaf(s[r], scale_log2, -offset));
    s[r] = p;
    u = u + p;
  }
  return u;
}

// P^T fragments of a block for its two 16-key k-steps: k-step k2 takes registers
// 8 k2 .. 8 k2 + 7 (keys 16 k2 + 8 (i/4) + 4 (l/32) + i%4, i = 0..7).
__device__ __forceinline__ void pack_p(const f32x16_t& p, bf16x8_t (&pf)[2]) {
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[k2][i] = (__bf16)p[8 * k2 + i];
  }
}

// The softmax part of a block update for this wave's rows: the row maximum of the
// block's (masked) scores s, the offset step, p = exp2(s c - offset) rounded to bf16
// into pf, l = alpha l + rowsum(p). Returns whether some row of the wave that already
// holds keys moved its offset (then O must be multiplied by alpha before the block's
// P*V is added; alpha is exactly 1 for every row that did not move).
template <int DO>
__device__ __forceinline__ bool block_softmax(f32x16_t& s, RowState<DO>& st, float scale_log2, bf16x8_t (&pf)[2],
                                              float& alpha) {
  const float mx = row_max(block_max(s));
  // The scale is positive, so the largest scaled score is the largest raw score, scaled.
  const float tile_max = mx * scale_log2;
  float m_new, offset;
  const bool move = softmax_step(st.m, tile_max, m_new, alpha, offset);
  const bool rescale = __any(move && st.m != kNegInf);
  const float u = exp_block(s, scale_log2, offset);
  st.l = alpha * st.l + row_sum(u);
  st.m = m_new;
  pack_p(s, pf);
  return rescale;
}

// ---- P*V for one block ------------------------------------------------------------
// V^T fragment of chunk c, k-step k2: head dims 32 c + (l % 32), keys (relative to the
// block) 16 k2 + 4 (l/32) + 0..3 and 16 k2 + 8 + 4 (l/32) + 0..3. Each transpose read
// serves 16 lanes: lane 4 r + q of the group reads 4 dims of key row r, and lane i of
// the group receives dim i of the 4 rows.
__device__ __forceinline__ bf16x4_t tr_read(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
}

__device__ __forceinline__ bf16x8_t cat(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D>
__device__ __forceinline__ bf16x8_t v_fragment(const lds_char_t* vst, const LaneOffsets<D>& lo, int c, int k2) {
  constexpr int R = Geom<D>::kRowBytes;
  const int c4 = c & 3;
  const int cb = (c >> 2) * 256 + k2 * 16 * R;
  return cat(tr_read(vst + lo.v[c4] + cb), tr_read(vst + lo.v[4 + c4] + cb));
}

// Output chunks C0 .. C0 + NCH - 1 (counted from the block's V rows at `vst`) +=
// V^T P^T, the two 16-key steps in order.
template <int D, int DO, int NCH, int C0>
__device__ __forceinline__ void pv_block(RowState<DO>& st, const lds_char_t* vst, const bf16x8_t (&pf)[2],
                                         const LaneOffsets<D>& lo) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    st.o[c] = mfma(v_fragment<D>(vst, lo, C0 + c, 0), pf[0], st.o[c]);
    st.o[c] = mfma(v_fragment<D>(vst, lo, C0 + c, 1), pf[1], st.o[c]);
  }
}

// ---- the pipelined block step of the prefill kernel ---------------------------------
// One scheduling region of a wave that owns NB N-blocks of 32 query slots: s_next[n] =
// S^T of the K block at ba.k for N-block n (if DO_S), the softmax of s_cur[n] (scores
// already masked) into p_cur[n] (if DO_SM), and O[n] += V^T p_prev[n]^T over the V
// block at ba.v (if DO_PV). Every K and V fragment read from LDS feeds NB MFMAs, which
// divides the LDS traffic per MFMA by NB. The parts are independent, so their
// instructions are interleaved by hand: step i issues the LDS reads of step i + kPf, the
// score MFMAs of k-step i, the P*V MFMAs i (chunk i / 2, key step i % 2) and a share of
// the softmax's vector work; a scheduling fence closes each step. The arithmetic of
// every part is exactly that of score_block, block_softmax and pv_block.
// LDS pointer from a byte address.
__device__ __forceinline__ const lds_char_t* lds_at(uint32_t addr) {
  return reinterpret_cast<const lds_char_t*>(static_cast<uintptr_t>(addr));
}

// LDS addresses of this lane's reads of one K block (score fragments) and of one V
// block (transpose reads), kept as loop-carried registers and moved from stage to
// stage by adding a constant. The score read of k-step kk is at
//   k[kk % 8] + (kk / 8) * 256,   k[i] = K block base + key (l % 32) * row bytes + ((i << 5) ^ k_sw),
// with k_sw = ((l / 32) ^ swizzle(key)) << 4: the swizzled chunk (2 (kk % 8) + (l / 32)) ^
// swizzle(key) equals 2 (kk % 8) ^ ((l / 32) ^ swizzle(key)) (the two terms share no bit)
// and 16 (kk / 8) is untouched by the 4-bit swizzle. The transpose reads keep their 8
// bases; every other part of a read's address is a compile-time offset in the
// instruction, so the loop spends no vector instruction on LDS addresses.
struct BlockAddr {
  uint32_t k[8];
  uint32_t v[8];
};

template <int D>
__device__ __forceinline__ void block_addr_init(BlockAddr& ba, const LaneOffsets<D>& lo, uint32_t kbase, uint32_t vbase,
                                                int lane) {
  const int key = lane & 31;
  const uint32_t k_row = kbase + (uint32_t)(key * Geom<D>::kRowBytes);
  const uint32_t k_sw = (uint32_t)(((lane >> 5) ^ chunk_swizzle<D>(key)) << 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) ba.k[i] = k_row + (((uint32_t)i << 5) ^ k_sw);
#pragma unroll
  for (int i = 0; i < 8; ++i) ba.v[i] = lo.v[i] + vbase;
}

// (A literal zero step costs nothing: the additions fold away.)
__device__ __forceinline__ void block_addr_move(BlockAddr& ba, int32_t dk, int32_t dv) {
#pragma unroll
  for (int i = 0; i < 8; ++i) ba.k[i] += (uint32_t)dk;
#pragma unroll
  for (int i = 0; i < 8; ++i) ba.v[i] += (uint32_t)dv;
}

template <int D>
__device__ __forceinline__ bf16x8_t k_fragment(const BlockAddr& ba, int kk) {
  return *reinterpret_cast<const lds_bf16x8_t*>(lds_at(ba.k[kk & 7]) + (kk >> 3) * 256);
}

// score_block over a K block given by absolute addresses.
template <int D>
__device__ __forceinline__ f32x16_t score_block_at(const BlockAddr& ba, const bf16x8_t (&qf)[Geom<D>::kKSteps]) {
  f32x16_t s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
  for (int kk = 0; kk < Geom<D>::kKSteps; ++kk) s = mfma(k_fragment<D>(ba, kk), qf[kk], s);
  return s;
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Softmax work in kSoftmaxParts ordered parts (see softmax_part).
constexpr int kSoftmaxParts = 18;

struct SoftmaxTemps {
  float mx;  // maxima (then, at the end, the partner lane's sum)
  float m_new;
  float offset;
  float u;   // this lane's sum of p, register order
  bool rescale;
};

// One part of a block's online softmax (the arithmetic of block_softmax). The parts run
// one or two matrix steps apart, and no part uses a result of the same part: within a
// part the wave issues without waiting on its own results, so the matrix instructions
// between the parts keep issuing. The exponentials run as a three-stage pipeline over
// parts 6 .. 15: the scaled score of values 2k, 2k + 1, their exp2 one part later and
// their addition to the row sum (in register order, as before) one part after that.
template <int DO>
__device__ __forceinline__ void softmax_part(int part, f32x16_t& s, RowState<DO>& st, SoftmaxTemps& t,
                                             float scale_log2, float& alpha, bf16x8_t (&pf)[2]) {
  if (part == 0) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, s[r]);
    t.mx = mx;
  } else if (part == 1) {
    float mx = s[8];
#pragma unroll
    for (int r = 9; r < 16; ++r) mx = fmaxf(mx, s[r]);
    t.m_new = mx;
  } else if (part == 2) {
    t.mx = fmaxf(t.mx, t.m_new);
  } else if (part == 3) {
    row_pair(t.mx, t.mx, t.m_new);
  } else if (part == 4) {
    t.mx = fmaxf(t.mx, t.m_new) * scale_log2;  // row_max of the lane maxima
  } else if (part == 5) {
    const bool move = softmax_step(st.m, t.mx, t.m_new, alpha, t.offset);
    t.rescale = __any(move && st.m != kNegInf);
    t.u = 0.0f;
  } else if (part < 16) {
    const int k = part - 6;
#pragma unroll
    for (int r = 2 * k - 4; r < 2 * k - 2; ++r) {
      if (r >= 0 && r < 16) t.u = t.u + s[r];
    }
#pragma unroll
    for (int r = 2 * k - 2; r < 2 * k; ++r) {
      if (r >= 0 && r < 16) s[r] = exp2_hw(s[r]);
    }
#pragma unroll
    for (int r = 2 * k; r < 2 * k + 2; ++r) {
      if (r < 16) s[r] = __builtin_fmaf(s[r], scale_log2, -t.offset);
    }
  } else if (part == 16) {
    row_pair(t.u, t.u, t.mx);
  } else {
    st.l = alpha * st.l + (t.u + t.mx);  // row_sum of the lane sums
    st.m = t.m_new;
    pack_p(s, pf);
  }
}

// LDS fragment reads run kPf steps ahead of their MFMAs: an LDS read takes about 100
// cycles, a step of two MFMAs (two N-blocks) 64 and of one MFMA (the 512-dim head) 32.
// A depth of 4 also fits the register file at both head sizes (and 5 at D = 256) but is
// no faster: the steps wait on the vector work under them, not on these reads. At
// D = 512 a depth of 3 measures about 0.6 % faster than 2 (fewer accumulator-register
// moves in the loop).
template <int D>
constexpr int prefetch_steps() { return 3; }

// LDS reads of the pipelined step as inline assembly. The compiler keeps inline
// assembly in program order, which keeps every fragment read kPf steps ahead of its
// MFMA (left to itself it issues all of a region's reads up front and runs out of
// registers); completion is tracked here with lgkmcnt, LDS operations completing in
// order. The results are kept as raw 32-bit words, and a transpose-read pair as its two
// halves, until the wait that names them: nothing may copy or repack a register whose
// read has not landed, and bf16 vectors built from two halves are repacked by the
// compiler.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct VPair {  // the two transpose reads of one A fragment of P*V
  u32x2_t lo, hi;
};

__device__ __forceinline__ u32x4_t asm_read_b128(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

__device__ __forceinline__ u32x2_t asm_read_tr(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

// The same with a compile-time byte offset in the instruction (at most 65535).
template <int OFF>
__device__ __forceinline__ u32x4_t asm_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

template <int OFF>
__device__ __forceinline__ u32x2_t asm_read_tr_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(const VPair& p) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(p.lo, p.hi, 0, 1, 2, 3));
}

// Wait until at most N LDS operations of this wave are in flight; the fragments are
// named as operands so no use (or copy) of them can move above the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& k) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(k) : "i"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(VPair& v) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v.lo), "+v"(v.hi) : "i"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& k, VPair& v) {
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(k), "+v"(v.lo), "+v"(v.hi) : "i"(N));
}

// Wait for the fragments of one pipeline step: the K fragment, the V fragment or both.
template <int N, bool K, bool V>
__device__ __forceinline__ void lds_wait_step(u32x4_t& kf, VPair& vf) {
  if constexpr (K && V) {
    lds_wait<N>(kf, vf);
  } else if constexpr (K) {
    lds_wait<N>(kf);
  } else {
    lds_wait<N>(vf);
  }
}

template <int D>
__device__ __forceinline__ u32x4_t k_read(const BlockAddr& ba, int kk) {
  const uint32_t a = ba.k[kk & 7];
  switch (kk >> 3) {
    case 0: return asm_read_b128_at<0>(a);
    case 1: return asm_read_b128_at<256>(a);
    case 2: return asm_read_b128_at<512>(a);
    default: return asm_read_b128_at<768>(a);
  }
}

// Transpose reads of V^T fragment (chunk c, key step k2): bases v[c % 4] and v[4 + c % 4],
// offset (c / 4) * 256 + k2 * 16 rows.
template <int D, int OFF>
__device__ __forceinline__ VPair v_read_off(const BlockAddr& ba, int c4) {
  return VPair{asm_read_tr_at<OFF>(ba.v[c4]), asm_read_tr_at<OFF>(ba.v[4 + c4])};
}

template <int D>
__device__ __forceinline__ VPair v_read(const BlockAddr& ba, int c, int k2) {
  constexpr int R16 = 16 * Geom<D>::kRowBytes;
  const int c4 = c & 3;
  switch (((c >> 2) << 1) | k2) {
    case 0: return v_read_off<D, 0>(ba, c4);
    case 1: return v_read_off<D, R16>(ba, c4);
    case 2: return v_read_off<D, 256>(ba, c4);
    case 3: return v_read_off<D, 256 + R16>(ba, c4);
    case 4: return v_read_off<D, 512>(ba, c4);
    case 5: return v_read_off<D, 512 + R16>(ba, c4);
    case 6: return v_read_off<D, 768>(ba, c4);
    default: return v_read_off<D, 768 + R16>(ba, c4);
  }
}

template <int D, int NB, bool DO_S, bool DO_SM, bool DO_PV>
__device__ __forceinline__ bool pipelined_step(RowState<D> (&st)[NB], f32x16_t (&s_next)[NB], f32x16_t (&s_cur)[NB],
                                               bf16x8_t (&p_cur)[NB][2], const bf16x8_t (&p_prev)[NB][2],
                                               float (&alpha)[NB], const BlockAddr& ba,
                                               const bf16x8_t (&qf)[NB][Geom<D>::kKSteps], float scale_log2) {
  constexpr int NSTEP = Geom<D>::kKSteps;  // = score k-steps = P*V key steps (D/32 chunks x 2)
  constexpr int kPf = prefetch_steps<D>();
  constexpr int RING = kPf + 1;
  constexpr int kReads = (DO_S ? 1 : 0) + (DO_PV ? 2 : 0);  // LDS reads per step
  SoftmaxTemps t[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) t[n].rescale = false;
  u32x4_t kf[RING];
  VPair vf[RING];
  if constexpr (DO_S) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_next[n][r] = 0.0f;
    }
  }
  auto issue = [&](int q) {
    if constexpr (DO_S) kf[q % RING] = k_read<D>(ba, q);
    if constexpr (DO_PV) vf[q % RING] = v_read<D>(ba, q >> 1, q & 1);
  };
#pragma unroll
  for (int q = 0; q < kPf && q < NSTEP; ++q) issue(q);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i + kPf < NSTEP) issue(i + kPf);
    // reads issued after step i's: those of steps i + 1 .. min(i + kPf, NSTEP - 1)
    constexpr int kAfterFull = kReads * kPf;
    if constexpr (kReads > 0) {
      u32x4_t& a = kf[i % RING];
      VPair& b = vf[i % RING];
      const int after = kReads * ((i + kPf < NSTEP ? i + kPf : NSTEP - 1) - i);
      if (after >= kAfterFull) {
        lds_wait_step<kAfterFull, DO_S, DO_PV>(a, b);
      } else if (after >= 2 * kReads) {
        lds_wait_step<2 * kReads, DO_S, DO_PV>(a, b);
      } else if (after >= kReads) {
        lds_wait_step<kReads, DO_S, DO_PV>(a, b);
      } else {
        lds_wait_step<0, DO_S, DO_PV>(a, b);
      }
    }
    if constexpr (DO_S) {
#pragma unroll
      for (int n = 0; n < NB; ++n) s_next[n] = mfma(as_bf16x8(kf[i % RING]), qf[n][i], s_next[n]);
    }
    if constexpr (DO_PV) {
#pragma unroll
      for (int n = 0; n < NB; ++n) st[n].o[i >> 1] = mfma(as_bf16x8(vf[i % RING]), p_prev[n][i & 1], st[n].o[i >> 1]);
    }
    if constexpr (DO_SM) {
      // parts [i * P / NSTEP, (i + 1) * P / NSTEP) of the NB interleaved softmaxes
      constexpr int P = kSoftmaxParts * NB;
#pragma unroll
      for (int q = (i * P) / NSTEP; q < ((i + 1) * P) / NSTEP; ++q)
        softmax_part<D>(q / NB, s_cur[q % NB], st[q % NB], t[q % NB], scale_log2, alpha[q % NB], p_cur[q % NB]);
    }
  }
  if constexpr (DO_SM && !DO_S && !DO_PV) {
    // softmax only: no reads, nothing to wait for
  }
  bool resc = false;
#pragma unroll
  for (int n = 0; n < NB; ++n) resc = resc || t[n].rescale;
  return resc;
}

// One region of the pipeline of a wave that owns two N-blocks, in which the softmax of
// a single N-block runs ("diagonal" placement: N-block 0's softmax of block j under
// the P*V of block j - 1, N-block 1's under the scores of block j + 1, so each region
// carries one softmax's vector work): S^T of the K block at ba into s[0..1] (if DO_S),
// O[n] += V^T p[n]^T over the V block at ba for both N-blocks (if DO_PV), and the
// softmax of N-block SMN's scores sm_s into sm_p (if DO_SM). Fragment reads, waits and
// the softmax parts are placed as in pipelined_step; the arithmetic of every part is
// that of score_block, block_softmax and pv_block.
template <int D, bool DO_S, bool DO_PV, bool DO_SM, int SMN>
__device__ __forceinline__ bool pipelined_step_diag(RowState<D> (&st)[2], f32x16_t (&s)[2], const bf16x8_t (&p)[2][2],
                                                    f32x16_t& sm_s, bf16x8_t (&sm_p)[2], float& sm_alpha,
                                                    const BlockAddr& ba, const bf16x8_t (&qf)[2][Geom<D>::kKSteps],
                                                    float scale_log2) {
  constexpr int NSTEP = Geom<D>::kKSteps;
  constexpr int kPf = prefetch_steps<D>();
  constexpr int RING = kPf + 1;
  constexpr int kReads = (DO_S ? 1 : 0) + (DO_PV ? 2 : 0);
  SoftmaxTemps t;
  t.rescale = false;
  u32x4_t kf[RING];
  VPair vf[RING];
  if constexpr (DO_S) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[n][r] = 0.0f;
    }
  }
  auto issue = [&](int q) {
    if constexpr (DO_S) kf[q % RING] = k_read<D>(ba, q);
    if constexpr (DO_PV) vf[q % RING] = v_read<D>(ba, q >> 1, q & 1);
  };
  if constexpr (kReads > 0) {
#pragma unroll
    for (int q = 0; q < kPf && q < NSTEP; ++q) issue(q);
  }
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if constexpr (kReads > 0) {
      if (i + kPf < NSTEP) issue(i + kPf);
      constexpr int kAfterFull = kReads * kPf;
      u32x4_t& a = kf[i % RING];
      VPair& b = vf[i % RING];
      const int after = kReads * ((i + kPf < NSTEP ? i + kPf : NSTEP - 1) - i);
      if (after >= kAfterFull) {
        lds_wait_step<kAfterFull, DO_S, DO_PV>(a, b);
      } else if (after >= 2 * kReads) {
        lds_wait_step<2 * kReads, DO_S, DO_PV>(a, b);
      } else if (after >= kReads) {
        lds_wait_step<kReads, DO_S, DO_PV>(a, b);
      } else {
        lds_wait_step<0, DO_S, DO_PV>(a, b);
      }
    }
    if constexpr (DO_S) {
#pragma unroll
      for (int n = 0; n < 2; ++n) s[n] = mfma(as_bf16x8(kf[i % RING]), qf[n][i], s[n]);
    }
    if constexpr (DO_PV) {
#pragma unroll
      for (int n = 0; n < 2; ++n) st[n].o[i >> 1] = mfma(as_bf16x8(vf[i % RING]), p[n][i & 1], st[n].o[i >> 1]);
    }
    if constexpr (DO_SM) {
#pragma unroll
      for (int q = (i * kSoftmaxParts) / NSTEP; q < ((i + 1) * kSoftmaxParts) / NSTEP; ++q)
        softmax_part<D>(q, sm_s, st[SMN], t, scale_log2, sm_alpha, sm_p);
    }
  }
  return t.rescale;
}

// out = bf16(O * (1 / l)); this lane writes dims 32 c + 8 g4 + 4 (l/32) + 0..3 of the
// slice that starts at orow.
template <int DO>
__device__ __forceinline__ void store_row(const RowState<DO>& st, uint16_t* orow, int lane) {
  const float inv = 1.0f / st.l;
#pragma unroll
  for (int c = 0; c < DO / 32; ++c) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(st.o[c][4 * g4 + e] * inv);
      *reinterpret_cast<bf16x4_t*>(orow + 32 * c + 8 * g4 + 4 * (lane >> 5)) = v;
    }
  }
}

// A row's partial result over one chunk of its keys (the split form): O as accumulated
// (fp32, not divided by l), this lane's dims 32 c + 8 g4 + 4 (l/32) + 0..3 of the slice
// at orow; with `ml`, lanes < 32 also write the row's offset m and sum l there.
template <int DO>
__device__ __forceinline__ void store_partial(const RowState<DO>& st, float* orow, float* ml, int lane) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int c = 0; c < DO / 32; ++c) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4_t v = {st.o[c][4 * g4], st.o[c][4 * g4 + 1], st.o[c][4 * g4 + 2], st.o[c][4 * g4 + 3]};
      *reinterpret_cast<f32x4_t*>(orow + 32 * c + 8 * g4 + 4 * (lane >> 5)) = v;
    }
  }
  if (ml && lane < kSlots) {
    ml[0] = st.m;
    ml[1] = st.l;
  }
}

// The same values as store_row, into one LDS row of the output tile (this lane's slot):
// dims 32 c + 8 g4 + 4 (l/32) + 0..3 at byte offset twice that.
template <int DO>
__device__ __forceinline__ void stage_row(const RowState<DO>& st, lds_char_t* trow, int lane) {
  const float inv = 1.0f / st.l;
#pragma unroll
  for (int c = 0; c < DO / 32; ++c) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(st.o[c][4 * g4 + e] * inv);
      *reinterpret_cast<lds_bf16x4_t*>(trow + 2 * (32 * c + 8 * g4 + 4 * (lane >> 5))) = v;
    }
  }
}

// ---- global memory -------------------------------------------------------------------
// Buffer descriptors: offsets at or beyond the record count read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

// A descriptor built from values the compiler may not know to be wave-uniform (they
// are, e.g. arguments of an out-of-line function): read from the first lane so that
// the descriptor lives in scalar registers, as the tile load requires.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(num_bytes);
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// Global -> LDS without registers: one wave instruction moves 64 x 16 bytes into the
// 1 KiB of LDS at `lds` (lane i fills bytes 16 i .. 16 i + 15); `lds` must be wave
// uniform. Issued as inline assembly so the compiler does not treat the in-flight
// load as a pending write to every LDS buffer (it would drain it before each LDS
// read); completion is tracked by the caller with s_waitcnt vmcnt and a barrier.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds),
      "v"(voff), "s"(rsrc)
      : "memory");
}

// s_waitcnt encodings (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
struct VmCnt {
  static_assert(N >= 0 && N < 64, "vmcnt");
  static constexpr int kImm = (N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8);
};

// Wait until at most N of this wave's vector memory loads are in flight and its LDS
// operations are done, then meet the other waves. Does not drain later loads.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt %0\n\ts_barrier" ::"i"(VmCnt<N>::kImm) : "memory");
}

// Meet the other waves once this wave's LDS operations are done (loads of later data
// may stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace g4
