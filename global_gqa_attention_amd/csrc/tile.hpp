// tile.hpp -- the one KV-tile update shared by the prefill and decode kernels.
//
// What it computes follows the attention work items of RL-Kernel issue #415
// (Gemma-4-31B-it RFC, section 5: sliding_attention_core, global_attention_core) under
// that page's section 4 numerical contract: fp32 accumulation, one fixed order of every
// reduction for a row, independent of which other rows share the work-group.
//
// Layout (gfx950, wave64):
//   * A wave owns 32 query slots (MFMA N). Scores are computed transposed,
//     S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read from LDS,
//     B = Q^T fragment kept in registers. Lane l then holds query slot l % 32 and 16
//     keys of the 32-key block: key(r) = 8 (r / 4) + 4 (l / 32) + (r % 4).
//   * Softmax statistics of a slot live in the two lanes l and l ^ 32; one
//     cross-lane exchange finishes each row reduction.
//   * O^T = V^T P^T with the same instruction: A = 32 head dims x 16 keys read from LDS
//     with the gfx950 transpose read (ds_read_b64_tr_b16), B = P^T taken straight from
//     the score registers. The 16 keys of one k-step are consumed in the permuted order
//     the score layout gives; that order is fixed, so every row sees one order.
//   * KV tiles are TILE_KEYS keys long and aligned to position 0 of the sequence, so a
//     row's tiles and their order depend only on its own position.
//   * LDS rows are D bf16 long (one key each) with 16-byte chunks XOR-swizzled by the
//     key index, which keeps both the score reads (16 lanes = 16 keys, same chunk) and
//     the transpose reads (4 keys x 4 chunks per 16 lanes) free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// The LDS address of a __shared__ object.
template <typename T>
__device__ __forceinline__ lds_char_t* lds_ptr(T* p) {
  return (lds_char_t*)(p);
}

constexpr int kWave = 64;
constexpr int kSlots = 32;      // query slots per wave (MFMA N)
constexpr int kKeyBlock = 32;   // keys per score block (MFMA M)
constexpr int kBlocks = 2;      // score blocks per KV tile
constexpr int kTileKeys = kKeyBlock * kBlocks;
constexpr int kWaves = 4;       // waves per work-group
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerGroup = kSlots * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane exchange with the lane 32 away (the other half of a query slot's row).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

template <int D>
struct Geom {
  static_assert(D == 64 || D == 128 || D == 256 || D == 512, "head dim");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;        // 16-byte chunks per key row
  static constexpr int kKSteps = D / 16;       // score k-steps over the head dim
  static constexpr int kDChunks = D / 32;      // 32-dim output chunks
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
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
// dims (the whole head, or one half of it when two work-groups share a query block).
template <int DO>
struct RowState {
  f32x16_t o[DO / 32];  // O^T chunk c: dim 32c + 8(r/4) + 4(l/32) + r%4 of the slice
  float m;                        // exponent offset (lazily updated running max, log2 units)
  float l;                        // running sum of exp2(score - m)
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
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[Geom<D>::kKSteps], const uint16_t* qrow,
                                       bool valid, int lane) {
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

// Per-lane LDS byte offsets. The swizzle only touches the low four bits of a chunk
// index and depends only on the low four bits of the key, so every read of a tile is
// one of 16 per-lane bases plus a compile-time offset.
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

// ---- S^T = K Q^T -------------------------------------------------------------------
// Every LDS access of the tile loop is issued as inline assembly and its completion
// tracked here (see the P*V section below for why): the compiler would otherwise treat
// each access as possibly aliasing the global->LDS loads of the next tile in flight and
// drain them first. LDS operations complete in order, so "at most N outstanding" after
// N newer reads of ours means the older ones are done, whatever else is in flight.
template <int IMM>
__device__ __forceinline__ bf16x8_t lds_read_b128(uint32_t addr) {
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

template <int N, int NB>
__device__ __forceinline__ void wait_frags(bf16x8_t (&f)[NB]) {
  if constexpr (NB == 1) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f[0]) : "i"(N));
  } else {
    static_assert(NB == 2, "one or two score blocks");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f[0]), "+v"(f[1]) : "i"(N));
  }
}

// K fragments of k-step KK for NB score blocks; addr[b][kk % 8] is the lane's address
// of block b's key row with the swizzled chunk 2 (kk % 8) + (l / 32).
template <int D, int NB, int KK>
__device__ __forceinline__ void issue_k(const uint32_t (&addr)[NB][8], bf16x8_t (&f)[NB]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) f[b] = lds_read_b128<(KK >> 3) * 256>(addr[b][KK & 7]);
}

// Score blocks += K Q^T for k-steps KK.. in ascending order; f0 holds step KK's
// fragments, f1 step KK + 1's (reads two steps ahead).
template <int D, int NB, int KK>
__device__ __forceinline__ void score_steps(f32x16_t (&s)[NB], const uint32_t (&addr)[NB][8],
                                            const bf16x8_t (&qf)[Geom<D>::kKSteps], bf16x8_t (&f0)[NB],
                                            bf16x8_t (&f1)[NB]) {
  constexpr int KS = Geom<D>::kKSteps;
  if constexpr (KK < KS) {
    bf16x8_t f2[NB];
    if constexpr (KK + 2 < KS) {
      issue_k<D, NB, KK + 2>(addr, f2);
      wait_frags<2 * NB, NB>(f0);
    } else if constexpr (KK + 1 < KS) {
      wait_frags<NB, NB>(f0);
    } else {
      wait_frags<0, NB>(f0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] = mfma(f0[b], qf[KK], s[b]);
    score_steps<D, NB, KK + 1>(s, addr, qf, f1, f2);
  }
}

// NB score blocks S^T = K Q^T (32 keys each), head dim in ascending 16-wide steps;
// block b's key rows start at LDS byte address base[b].
template <int D, int NB>
__device__ __forceinline__ void score_blocks(f32x16_t (&s)[NB], const uint32_t (&base)[NB], const LaneOffsets<D>& lo,
                                             const bf16x8_t (&qf)[Geom<D>::kKSteps]) {
  uint32_t addr[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) addr[b][k8] = base[b] + lo.k[k8];
  }
  bf16x8_t f0[NB], f1[NB];
  issue_k<D, NB, 0>(addr, f0);
  issue_k<D, NB, 1>(addr, f1);
  score_steps<D, NB, 0>(s, addr, qf, f0, f1);
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

// Hide the keys of one score block outside the row's range (score -> -inf). The key of
// register r is key_pos0 + 8 (r/4) + (r%4), key_pos0 = tile start + 32 b + 4 (l/32).
__device__ __forceinline__ void mask_block(f32x16_t& s, int key_pos0, RowBounds rb) {
  const int above = rb.hi - key_pos0;  // visible iff offset <= above
  const int below = rb.lo - key_pos0;  // ... and offset >= below
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + (r & 3);
    s[r] = (off <= above && off >= below) ? s[r] : kNegInf;
  }
}

// Largest of this lane's 16 raw scores of one block.
__device__ __forceinline__ float block_max(const f32x16_t& s) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  return mx;
}

// Threshold of the lazy max update, in log2 units: the exponent offset of a row only
// moves when a tile's largest score exceeds it by more than this, so probabilities stay
// <= 2^8 before normalisation and most tiles need no rescale of O at all.
constexpr float kRescaleThreshold = 8.0f;

// Decide a row's exponent offset for this tile. m_old is the offset in use (-inf before
// the first visible key). Returns the new offset m_new, the factor alpha that rescales
// the old (l, O) (exactly 1 when the offset stays), and `offset`, the value subtracted
// from the scores (0 while the row has seen no visible key, so hidden keys give
// exp2(-inf) = 0). A tile without visible keys leaves (m, l, O) bit-for-bit unchanged.
__device__ __forceinline__ bool softmax_step(float m_old, float tile_max, float& m_new, float& alpha,
                                             float& offset) {
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

// P^T fragments of one block for the two 16-key k-steps: k-step k2 takes registers
// 8 k2 .. 8 k2 + 7 (keys 16 k2 + 8 (i/4) + 4 (l/32) + i%4, i = 0..7).
__device__ __forceinline__ void pack_p(const f32x16_t& p, bf16x8_t (&pf)[2]) {
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[k2][i] = (__bf16)p[8 * k2 + i];
  }
}

// Multiply every O accumulator of the state by alpha (this lane's slot factor).
template <int DO>
__device__ __forceinline__ void rescale_o(RowState<DO>& st, float alpha) {
#pragma unroll
  for (int c = 0; c < DO / 32; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[c][r] = st.o[c][r] * alpha;
  }
}

// ---- P*V -------------------------------------------------------------------------
// V^T fragment of chunk c, block b, k-step k2: head dims 32 c + (l % 32), keys
// (relative to the tile) kb + 4 (l/32) + 0..3 and kb + 8 + 4 (l/32) + 0..3,
// kb = 32 b + 16 k2. Each transpose read serves 16 lanes: lane 4 r + q of the group
// reads 4 dims of key row r, and lane i of the group receives dim i of the 4 rows.
//
// The transpose reads are issued as inline assembly: the compiler treats the builtin
// form as aliasing the in-flight global->LDS loads of the next tile and would wait for
// them before every read. Completion is tracked here instead: LDS operations finish in
// order, so after issuing the next chunk's 8 reads, "at most 8 outstanding" means this
// chunk's reads are done whatever else is in flight. The wait names the fragments as
// operands, so no use of them can be scheduled before it.
template <int IMM>
__device__ __forceinline__ bf16x4_t tr_read(uint32_t addr) {
  bf16x4_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_lds(bf16x8_t (&f)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]) : "i"(N));
}

__device__ __forceinline__ bf16x8_t cat(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Issue the 8 reads of chunk C: fragments (b, k2) = (0,0), (0,1), (1,0), (1,1).
// addr[part * 4 + c4] is this lane's LDS address for key part `part` and c % 4 == c4.
template <int D, int C>
__device__ __forceinline__ void issue_chunk(const uint32_t (&addr)[8], bf16x8_t (&f)[4]) {
  static_assert(kBlocks == 2, "four fragments per chunk");
  constexpr int R = Geom<D>::kRowBytes;
  constexpr int c4 = C & 3;
  constexpr int cb = (C >> 2) * 256;
  f[0] = cat(tr_read<0 * R + cb>(addr[c4]), tr_read<0 * R + cb>(addr[4 + c4]));
  f[1] = cat(tr_read<16 * R + cb>(addr[c4]), tr_read<16 * R + cb>(addr[4 + c4]));
  f[2] = cat(tr_read<32 * R + cb>(addr[c4]), tr_read<32 * R + cb>(addr[4 + c4]));
  f[3] = cat(tr_read<48 * R + cb>(addr[c4]), tr_read<48 * R + cb>(addr[4 + c4]));
}

// Local O^T chunk C (chunk C0 + C counted from lds_v) += V^T P^T over the tile's keys
// (blocks, then k-steps, ascending), with the reads of the next chunk in flight.
template <int D, int DO, int C0, int C>
__device__ __forceinline__ void pv_chunks(RowState<DO>& st, const uint32_t (&addr)[8],
                                          const bf16x8_t (&pf)[kBlocks][2], bf16x8_t (&cur)[4]) {
  if constexpr (C < DO / 32) {
    bf16x8_t nxt[4];
    if constexpr (C + 1 < DO / 32) {
      issue_chunk<D, C0 + C + 1>(addr, nxt);
      wait_lds<8>(cur);
    } else {
      wait_lds<0>(cur);
    }
    st.o[C] = mfma(cur[0], pf[0][0], st.o[C]);
    st.o[C] = mfma(cur[1], pf[0][1], st.o[C]);
    st.o[C] = mfma(cur[2], pf[1][0], st.o[C]);
    st.o[C] = mfma(cur[3], pf[1][1], st.o[C]);
    if constexpr (C + 1 < DO / 32) pv_chunks<D, DO, C0, C + 1>(st, addr, pf, nxt);
  }
}

// O^T chunks C0 .. C0 + DO/32 - 1 (counted from lds_v, which must sit a multiple of
// 16 chunks of 16 bytes into the row so the swizzle is unchanged) += V^T P^T.
template <int D, int DO, int C0 = 0>
__device__ __forceinline__ void pv_update(RowState<DO>& st, const lds_char_t* lds_v, const bf16x8_t (&pf)[kBlocks][2],
                                          const LaneOffsets<D>& lo) {
  const uint32_t base = (uint32_t)(uintptr_t)lds_v;
  uint32_t addr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) addr[i] = base + lo.v[i];
  bf16x8_t cur[4];
  issue_chunk<D, C0>(addr, cur);
  pv_chunks<D, DO, C0, 0>(st, addr, pf, cur);
}

// The whole tile update for one wave that owns all of the tile's work:
// scores, mask, softmax statistics, rescale and P*V.
//
// kRescale = false is the fast form: it returns false, before touching the state, when
// some row of the wave that already holds keys would move its exponent offset (the
// caller then redoes the tile with kRescale = true and stays on that form). A row's
// first offset (from -inf) needs no rescale: its l and O are still exactly zero.
// Rows whose offset stays have alpha == 1 exactly, so multiplying only when some row
// moved changes no bit of any row.
template <int D, int DO, bool kRescale>
__device__ __forceinline__ bool tile_update(RowState<DO>& st, const lds_char_t* lds_k, const lds_char_t* lds_v,
                                            const LaneOffsets<D>& lo, const bf16x8_t (&qf)[Geom<D>::kKSteps],
                                            int tile_pos0, RowBounds rb, float scale_log2, bool need_mask,
                                            int lane) {
  f32x16_t s[kBlocks];
  uint32_t kbase[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) kbase[b] = (uint32_t)(uintptr_t)lds_k + b * kKeyBlock * Geom<D>::kRowBytes;
  score_blocks<D, kBlocks>(s, kbase, lo, qf);
  if (need_mask) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) mask_block(s[b], tile_pos0 + b * kKeyBlock + 4 * (lane >> 5), rb);
  }
  float mx = block_max(s[0]);
#pragma unroll
  for (int b = 1; b < kBlocks; ++b) mx = fmaxf(mx, block_max(s[b]));
  mx = fmaxf(mx, swap_halves(mx));
  // The scale is positive, so the largest scaled score is the largest raw score, scaled.
  const float tile_max = mx * scale_log2;
  float m_new, alpha, offset;
  const bool move = softmax_step(st.m, tile_max, m_new, alpha, offset);
  const bool rescale = __any(move && st.m != kNegInf);
  if constexpr (!kRescale) {
    if (rescale) return false;
  }
  float u[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) u[b] = exp_block(s[b], scale_log2, offset);
  float half = u[0];
#pragma unroll
  for (int b = 1; b < kBlocks; ++b) half = half + u[b];
  const float total = half + swap_halves(half);
  st.l = alpha * st.l + total;
  st.m = m_new;
  bf16x8_t pf[kBlocks][2];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) pack_p(s[b], pf[b]);
  if constexpr (kRescale) {
    if (rescale) rescale_o<DO>(st, alpha);
  }
  pv_update<D, DO>(st, lds_v, pf, lo);
  return true;
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

// ---- tile loads: global -> LDS without registers (buffer_load ... lds) -------------
// One wave instruction moves 64 x 16 bytes into 1 KiB of contiguous LDS; lane i fills
// physical chunk i of that KiB, so it fetches the logical chunk the swizzle puts there.
// Offsets at or beyond the descriptor's record count read as zero.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// Instructions per wave for one K (or V) tile, and where lane `lane` of instruction i
// of wave `wave` lands: tile row and logical 16-byte chunk.
template <int D>
struct TileLoadMap {
  static constexpr int kInstr = Geom<D>::kTileBytes / 1024 / kWaves;
  int row[kInstr];
  int chunk_bytes[kInstr];
};

template <int D>
__device__ __forceinline__ TileLoadMap<D> tile_load_map(int wave, int lane) {
  static_assert((Geom<D>::kTileBytes / 1024) % kWaves == 0, "tile split");
  TileLoadMap<D> m;
#pragma unroll
  for (int i = 0; i < TileLoadMap<D>::kInstr; ++i) {
    const int j = wave + kWaves * i;
    const int byte = j * 1024 + lane * 16;
    m.row[i] = byte / Geom<D>::kRowBytes;
    const int phys = (byte % Geom<D>::kRowBytes) >> 4;
    m.chunk_bytes[i] = (phys ^ chunk_swizzle<D>(m.row[i])) << 4;
  }
  return m;
}

// Issue one tile's loads; voff[i] is this lane's byte offset for instruction i
// (kOutOfRange reads zero). `wave` must be wave-uniform (it sets the LDS address).
template <int D>
__device__ __forceinline__ void load_tile(lds_char_t* lds_tile, __amdgpu_buffer_rsrc_t rsrc,
                                          const uint32_t (&voff)[TileLoadMap<D>::kInstr], int wave) {
#pragma unroll
  for (int i = 0; i < TileLoadMap<D>::kInstr; ++i) {
    const int j = wave + kWaves * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds_tile + j * 1024), 16, (int)voff[i], 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_tile_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Work-group barrier for exchanges through LDS while tile loads are in flight: waits
// only for this wave's LDS operations (so its exchange writes are visible), not for
// the global->LDS loads of later tiles, which the compiler's own barrier would drain.
__device__ __forceinline__ void exchange_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exchange-area accesses (inline assembly for the reason given with the score reads).
// Stores are made visible to the other waves by exchange_barrier(); loads return with
// their data in place.
template <int IMM>
__device__ __forceinline__ void lds_store_f32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(IMM));
}

template <int IMM>
__device__ __forceinline__ void lds_store_b128(uint32_t addr, bf16x8_t v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(IMM));
}

template <int I0, int I1>
__device__ __forceinline__ void lds_load2_f32(uint32_t addr, float& x0, float& x1) {
  asm volatile(
      "ds_read_b32 %0, %2 offset:%3\n\t"
      "ds_read_b32 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1)
      : "v"(addr), "i"(I0), "i"(I1));
}

template <int I0, int I1, int I2, int I3>
__device__ __forceinline__ void lds_load4_b128(uint32_t addr, bf16x8_t& x0, bf16x8_t& x1, bf16x8_t& x2,
                                               bf16x8_t& x3) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(addr), "i"(I0), "i"(I1), "i"(I2), "i"(I3));
}


}  // namespace g4
