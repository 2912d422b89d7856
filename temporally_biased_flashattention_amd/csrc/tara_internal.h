// Internal interface between the C ABI host code (tara_host.cpp) and the
// gfx950 kernels (tara_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "tara.h"

namespace tara {

constexpr int kBlockK = 64;          // keys per key tile (all paths)
constexpr int kMaxParts = 64;        // == TARA_MAX_PARTITIONS
constexpr int kMaxPictures = 16;     // == TARA_MAX_PICTURES
constexpr int kMaxBindings = 4;      // == TARA_MAX_BINDINGS
constexpr int kMaxListTiles = 16384; // key tiles a three-term pass can list (N <= 2^20)

// What one pass of the attention kernel computes.
//  FUSED   all keys, final O and LSE
//  RANGE   key range [kr[p], kr[p+1]) of partition p = blockIdx.y -> O_p, LSE_p
//  TERM_A/B/C  the three non-negative contributions of the Flash Partitions
//          evaluation ("Three backends"), each a partition (p = 0, 1, 2):
//          A: keys that are not biased guide keys, normal logits;
//          B: biased guide keys, target rows at -cap (other rows unbiased);
//          C: biased guide keys x target rows, weight e^s (e^-penalty - e^-cap),
//             i.e. logit s + ln(e^-penalty - e^-cap) (-inf past the saturation gap).
//          A pass visits only the key tiles that hold keys of its term (and, for
//          C, guide times within the saturation gap of the workgroup's rows).
enum : int { PASS_FUSED = 0, PASS_RANGE = 1, PASS_TERM_A = 2, PASS_TERM_B = 3, PASS_TERM_C = 4 };

// Variants of the fused bf16 pass: plain; 8-bit Q.K; the dense-bias baseline
// (bias read per element from a materialised [B][N][npad] fp32 tensor).
enum : int { ATTN_PLAIN = 0, ATTN_QK8 = 1, ATTN_DENSE_BIAS = 2 };

// Kind of a key tile, from the per-key encodings (see MetaArgs):
//  PLAIN   no key of the tile can carry a bias term
//  GUIDE   every key is a biased guide key; lo/hi = min/max time (s)
//  PICTURE every key is a key of the same bound picture `pic`: the bias of a
//          row is its gain-table entry for that picture
//  MIXED   anything else (per-element bias)
// KT_HAS_PICTURE is or-ed into kind when some key of the tile is a bound
// picture key (the per-element path then reads the gain table).
enum : int { KT_PLAIN = 0, KT_GUIDE = 1, KT_PICTURE = 2, KT_MIXED = 3, KT_CLASS = 3, KT_HAS_PICTURE = 4 };

struct __attribute__((aligned(16))) KeyTileSummary {
  int kind;
  float lo;
  float hi;
  int pic;      // picture id of a PICTURE tile, else -1
};

// Per-token encodings written by the metadata kernel. The temporal rule is
// evaluated in log2 units: with sigma = sqrt(strength * log2 e) / falloff,
//   penalty * log2 e = min(max(|tq - tk| * sigma - w, 0)^2, cap2),
// w = window * sigma, cap2 = cap * log2 e. Times stay in seconds so the gap
// |tq - tk| is rounded relative to itself, not to the absolute times.
//   tq[b][n]  time of a biased (target) query, NaN otherwise
//   tk[b][n]  time of a biased (guide) key, NaN otherwise (n < npad)
//   kp[b][n]  picture id of a bound picture key, -1 otherwise (n < npad)
//   gt[b][n][P]  summed log2 gains of a target query for each picture id,
//             sum_j m_j * log2 gain_j,p (0 for other queries); P = npics
// A NaN time makes the penalty 0 (fmaxf(NaN, 0) = 0), which is how unbiased
// query/key pairs drop out of the per-element formula.
struct MetaArgs {
  const uint8_t* seg;
  const float* time;
  const int16_t* pic;
  const float* mask;       // [nbind][...][N] or NULL; planes mask_plane elements apart
  int64_t mask_plane;
  int B, N, npad, nkt;
  int bias_active, binding_active, num_pictures, nbind;
  float lg2gain[kMaxBindings][kMaxPictures];
  float* tq;
  float* tk;
  int* kp;
  float* gt;              // [B][N][num_pictures] (binding active only)
  KeyTileSummary* ksum;   // [B][nkt]
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;           // fp32 path reads V directly
  const __bf16* vt;        // bf16 path: V as [B*H][D][npad], keys contiguous
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  void* o;                 // fused: final O (input dtype)
  float* lse;              // fused: final LSE [B][H][N]
  float* opart;            // partitioned: O_p fp32 [P][B][H][prows][D]
  float* lsepart;          // partitioned: LSE_p [P][B][H][prows]
  int prow0, prows;        // rows [prow0, prow0 + prows) of each (b, h) that O_p / LSE_p hold
                           // (their N above is prows; 0 and N but for the fused pass's tail)
  int B, H, N, npad, nkt, nqb;
  int qr0, qr1;            // query rows of this launch: [qr0, qr1) (all: 0, N); nqb covers them
  const float* tq;
  const float* tk;
  const int* kp;
  const float* gt;
  int npics;               // row length of gt
  const KeyTileSummary* ksum;
  const float* kmax;       // bf16 path: [B*H][nkt] max |k| per key tile
  const uint8_t* k8;       // 8-bit Q.K: FP8 E4M3 keys [B*H][npad][D]
  const float* ks;         // 8-bit Q.K: power-of-two scale per key tile [B*H][nkt]
  const float* dbias;      // dense-bias baseline: [B][N][npad] bias in log2 units
  float c;                 // softmax_scale * log2 e
  float sigma;             // sqrt(strength * log2 e) / falloff  (1/s)
  float w;                 // window * sigma
  float cap2;              // cap * log2 e
  float window;            // seconds: gaps <= window carry no penalty
  float dsat;              // seconds: gaps >= window + falloff*sqrt(cap/strength) carry exactly cap
  float corr0;             // log2(1 - 2^-cap2): term C's logit offset for gaps inside the window
  int elem_all;            // nonzero: every key tile takes the per-element bias (no tile classes)
  int nparts;
  int kr[kMaxParts + 1];   // partition key offsets (fused: {0, N})
};

struct MergeArgs {
  const float* opart;
  const float* lsepart;
  void* o;
  float* lse;
  int64_t o_sb, o_sh, o_sn;
  int B, H, N, D, nparts;
  int row0, rows;          // merge rows [row0, row0 + rows) of each (b, h); partials hold rows - row0
};

hipError_t launch_meta(const MetaArgs& a, hipStream_t s);
hipError_t launch_vtranspose(const __bf16* v, int64_t sb, int64_t sh, int64_t sn, __bf16* vt,
                             int B, int H, int N, int npad, int D, hipStream_t s);
hipError_t launch_knorm(const __bf16* k, int64_t sb, int64_t sh, int64_t sn, float* kmax, int B, int H, int N,
                        int nkt, int D, hipStream_t s);
hipError_t launch_kquant(const __bf16* k, int64_t sb, int64_t sh, int64_t sn, uint8_t* k8, float* ks, float* kmax,
                         int B, int H, int N, int npad, int nkt, int D, hipStream_t s);
// Block of query rows per workgroup of the bf16 attention kernel.
int attn_bf16_block_q(int D);
int attn_bf16_grid(const AttnArgs& a);
hipError_t launch_attn_bf16(const AttnArgs& a, int D, int pass, int variant, hipStream_t s);
hipError_t launch_dense_bias(const AttnArgs& a, float* out, hipStream_t s);
int attn_f32_block_q(int D);
hipError_t launch_attn_f32(const AttnArgs& a, int D, int pass, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, bool bf16_out, hipStream_t s);

// Tile-class counts (debug readback, FUSED and RANGE passes): (row, key tile)
// pairs per bias class, per batch element and group of 32 query rows.
enum : int { TC_PLAIN = 0, TC_SATURATED = 1, TC_WINDOW = 2, TC_PICTURE = 3, TC_ELEM = 4, TC_COUNT = 5 };
inline int tile_stats_groups(int N) { return (N + 31) / 32; }
hipError_t launch_tile_stats(const AttnArgs& a, int pass, unsigned* counts, hipStream_t s);

// ----------------------------------------------------------- host side
// One tara_attn_fwd call, its arguments checked by make_call. Metadata rows
// of consecutive batch elements are N apart; mask planes mask_plane apart.
struct Call {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  tara_dtype_t dtype;
  int B, H, N, D;
  int64_t qs[3], ks[3], vs[3], os[3];
  const uint8_t* seg;
  const float* time;
  const int16_t* pic;
  const float* mask;
  int64_t mask_plane;
  const tara_params_t* p;
  // a fused call's tail split, planned for the whole call (B, H) and kept by
  // its sub-calls, so that they run the same passes per head: query blocks
  // per (b, h) in the fused pass, key ranges of the rest (0: none), first row
  // of the rest
  int tail_m, tail_parts, tail_row0;
};
// Checks the arguments of tara_attn_fwd (everything but the workspace) and
// fills c; a nonzero status (with the thread's last error set) on failure.
int make_call(Call& c, const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int B,
              int H, int N, int D, const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
              const int64_t o_str[3], const uint8_t* seg_type, const float* token_time, const int16_t* picture_id,
              const float* mask_weight, const tara_params_t* p);
// Workspace bytes of the call's shape.
size_t call_workspace(const Call& c);
// Batch element b, heads [h0, h0 + hc) of c, as a call of its own (B = 1).
Call sub_call(const Call& c, int b, int h0, int hc);
// Enqueues the call on stream with a workspace of call_workspace(c) bytes
// (256-byte aligned). run_meta = false reuses the metadata encodings the
// workspace already holds for the same batch element. debug: record the
// timing events and honour TARA_TILE_STATS / TARA_LOG (the tile readback
// synchronises the stream). Fills *info.
int enqueue_call(const Call& c, char* ws, bool run_meta, bool debug, hipStream_t stream, tara_run_info_t* info);
void set_last_info(const tara_run_info_t& info);
void set_empty_info(const Call& c);
int set_error(int status, const std::string& msg);

}  // namespace tara
