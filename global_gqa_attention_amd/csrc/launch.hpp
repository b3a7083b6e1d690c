// launch.hpp -- host-side launcher interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g4 {

// cos and sin of the RoPE angle of rotated pair i at position pos: the frequency
// theta^(-2i/F) and the product pos * frequency in fp64; the angle reduced to [-pi, pi] in
// fp64 (two-part 2 pi with fused multiply-adds, error far below fp32 resolution), split
// into an fp32 head and tail; cos/sin(head + tail) from fp32 cos/sin of the head and a
// first-order correction in the tail, i.e. to within about an fp32 rounding of the fp64
// values. (The q/k prologue and the prefill's own q prologue share it.)
__device__ __forceinline__ void rope_cos_sin(int pos, int i, double theta, int freq_dim, float& c, float& s) {
  constexpr double kTwoPiHi = 6.283185307179586232;    // 2 pi rounded to fp64
  constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2 pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double inv_freq = pow(theta, -2.0 * (double)i / (double)freq_dim);
  const double ang = (double)pos * inv_freq;
  const double k = rint(ang * kInvTwoPi);
  const double red = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
  const float hi = (float)red;
  const float lo = (float)(red - (double)hi);
  float sh, ch;
  sincosf(hi, &sh, &ch);
  c = fmaf(-sh, lo, ch);
  s = fmaf(ch, lo, sh);
}

struct PrologueArgs {
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  uint16_t* k_out;
  const uint16_t* v_in;
  uint16_t* v_out;
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  const int32_t* positions;
  const int64_t* kv_dst_row;
  int64_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t rope_dims;
  int32_t rope_freq_dim;
  int32_t pair_offset;  // partner of rotated dim i (< R/2) is i + pair_offset
  double rope_theta;
  float rms_eps;
  int32_t v_norm;  // 1: v rows stored as their unit RMS norm; 0: copied raw
};

// The split form (global layers): a row's keys go in chunks of `keys` positions aligned
// to position 0; each chunk's work-group writes the row's partial result over that
// chunk (O unscaled, offset m, sum l), and the merge kernel combines a row's chunks in
// ascending order. A row whose keys lie in one chunk is written whole, as without the
// split. Partial p = ((b * rows + i) * Hq + h) * chunks + c for row i of sequence b
// (its position minus that of the call's first row), query head h, chunk c.
struct SplitArgs {
  int32_t keys;    // positions per chunk (0: no split)
  int32_t chunks;  // chunk slots per row in the partial layout
  int32_t rows;    // row slots per sequence in the partial layout
  float* part_o;   // [partials, D] fp32
  float* part_ml;  // [partials, 2] fp32: offset m, sum l
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;  // == k when one tensor is both K and V
  uint16_t* out;
  const int32_t* seq_start;  // first q / out row of each sequence (chunk)
  const int32_t* seq_len;    // query rows of each sequence (chunk)
  const int32_t* q_pos0;     // position of each chunk's first row (null: 0)
  const int64_t* kv_row0;    // row of position 0 (slot 0) of each sequence's keys (null: seq_start)
  int32_t kv_slots;          // keys of position p at row kv_row0 + p mod kv_slots (0: no wrap)
  const int32_t* last_key;   // per q row: position of the last key the row sees (null: its own)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t window;
  int32_t num_qblocks;  // query blocks of the longest sequence
  int32_t batch;
  float scale_log2;  // softmax scale * log2(e)
  SplitArgs split;
  // (the q prologue inside the prefill: q holds the raw rows, normed and rotated as the
  // work-group stages them, with the prologue's arithmetic)
  const uint16_t* q_norm_w;
  const int32_t* positions;  // per q row
  int32_t rope_dims;
  int32_t rope_freq_dim;
  int32_t pair_offset;
  double rope_theta;
  float rms_eps;
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;  // == k_cache when one tensor is both K and V
  uint16_t* out;
  const int64_t* cache_row0;
  const int32_t* ctx_len;
  const int32_t* schedule;  // may be null
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t window;
  int32_t cache_slots;
  int32_t batch;
  float scale_log2;
  SplitArgs split;
};

// The merge of the split form: row i of sequence b (i < nrows[b], or one row) sits at
// position (pos_ref ? pos_ref[b] : 0) + pos_bias + i and is written to packed out row
// (out_row0 ? out_row0[b] : b) + i; rows with keys in one chunk are skipped.
struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  const int32_t* out_row0;
  const int32_t* nrows;
  const int32_t* pos_ref;
  int32_t pos_bias;
  int32_t num_q_heads;
  int32_t batch;
  int32_t rows;
  int32_t chunks;
  int32_t split_keys;
  int32_t row_skip;  // rows 0 .. row_skip - 1 of every sequence have one chunk (not launched)
};

struct BackwardArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;  // == k when one tensor is both K and V
  const uint16_t* out;   // the forward output
  const uint16_t* dout;  // the gradient of the loss with respect to out
  uint16_t* dq;
  uint16_t* dk;  // with one tensor as K and V: the gradient of both roles
  uint16_t* dv;  // null when one tensor is both K and V
  float* lse;    // [T, Hq] log2 of each row's sum of exp(score) (written)
  float* delta;  // [T, Hq] each row's dO . out (written)
  const int32_t* seq_start;
  const int32_t* seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t window;
  int32_t num_qblocks;  // 128-row query blocks of the longest sequence
  int32_t num_kblocks;  // 128-key blocks of the longest sequence
  int32_t batch;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
};

struct LaunchShape {
  int32_t block_q;
  int32_t block_k;
  int32_t waves;
  const char* kernel_name;
};

// Query rows (position x head) per prefill work-group for a head dim and K/V form; the
// narrow form (one N-block per wave) serves grids too small to fill the GPU.
int prefill_rows_per_group(int head_dim, bool k_eq_v, bool narrow);

hipError_t launch_prologue(int head_dim, const PrologueArgs& a, hipStream_t stream);
hipError_t launch_prefill(int head_dim, bool k_eq_v, bool narrow, const PrefillArgs& a, hipStream_t stream,
                          LaunchShape* shape);
hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, hipStream_t stream, LaunchShape* shape);
// The prefill of raw q rows, the q prologue inside (head dim 512, K=V; a.q_norm_w, a.positions
// and the RoPE fields set).
hipError_t launch_prefill_qp(const PrefillArgs& a, hipStream_t stream, LaunchShape* shape);
// The library's own partial-result buffer for callers that cannot allocate (one array per
// GPU, held for the life of the process; calls that overlap on one GPU race on it).
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
// The device address of the current GPU's array (looked up once per device).
hipError_t scratch_address(void** ptr);

// The split form (a.split.keys > 0): the chunk work-groups (no narrow form), then the merge.
hipError_t launch_prefill_split(int head_dim, bool k_eq_v, const PrefillArgs& a, const MergeArgs& m,
                                hipStream_t stream, LaunchShape* shape);
hipError_t launch_decode_split(int head_dim, bool k_eq_v, const DecodeArgs& a, const MergeArgs& m,
                               hipStream_t stream, LaunchShape* shape);
// The backward's two launches on `stream`: dQ with the row statistics, then dK and dV.
hipError_t launch_backward(int head_dim, bool k_eq_v, const BackwardArgs& a, hipStream_t stream);

}  // namespace g4
