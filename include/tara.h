/*
 * tara.h - C ABI of the MI355X (gfx950) TARA attention library (libtara.so).
 *
 * TARA ("TARA: Native Temporal Alignment for MiniMax H3 References", section
 * "The temporal rule") is scaled-dot-product attention over one packed token
 * sequence (output video, selected motion-guide video, reference pictures,
 * text, ...) in which only logits from output-video (target) queries to guide
 * keys are lowered by a temporal penalty
 *
 *     dt      = |t_query - t_key|                                    (seconds)
 *     penalty = min(strength * (max(dt - window, 0) / falloff)^2, cap)
 *     logit   = (Q . K) * softmax_scale - penalty
 *
 * and, with reference binding on ("BFS H3 Reference Attention Binding
 * (Experimental)", section "The exact rule"), logits from target queries with
 * mask weight m to keys of Picture i gain m * ln(gain_i); chained bindings add
 * their terms (section "Common issues"): sum_j m_j * ln(gain_j,i). Every other logit is
 * plain (Q . K) * softmax_scale. One non-causal softmax runs over all keys of
 * the sequence. The library returns O and the natural-log log-sum-exp (LSE) of
 * each query row's final logits.
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device memory of the current device; host
 *    pointers are marked "host". The caller owns every buffer; the library never
 *    allocates, frees or retains device memory between calls.
 *  - All work is enqueued asynchronously on `stream` (NULL = default stream);
 *    inputs and workspace must stay valid until the stream has passed the call.
 *  - Return value: TARA_OK (0) or a negative tara_status_t. Argument errors are
 *    detected on the host before any device work is enqueued, so a failing call
 *    leaves outputs untouched. tara_last_error() gives the detail (per thread).
 *  - Thread safety: calls from several host threads are safe; concurrent calls
 *    on one stream serialise in stream order.
 */
#ifndef TARA_H_
#define TARA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* tara_stream_t; /* a hipStream_t */

/* Segment codes of seg_type[]: which part of the packed sequence a token is.
 * TARGET = output video (the only biased queries); GUIDE = the motion video
 * selected by motion_video_index (the only temporally penalised keys; "Wiring
 * it" section); PICTURE = a native reference picture (binding keys);
 * OTHER = text, reference audio, other videos: plain attention both ways. */
enum {
  TARA_SEG_TARGET = 0,
  TARA_SEG_GUIDE = 1,
  TARA_SEG_PICTURE = 2,
  TARA_SEG_OTHER = 3
};

typedef enum { TARA_BF16 = 0, TARA_FP32 = 1 } tara_dtype_t;

/* FUSED: one streaming pass over all keys.
 * PARTITIONED: the keys are split into num_partitions contiguous ranges, each
 * range is attended on its own with its own LSE, and the ranges are merged
 * exactly by log-sum-exp (the LSE-merging evaluation of the "Three backends"
 * section).
 * THREE_TERM: the Flash Partitions evaluation of that section, read as three
 * non-negative contributions, each attended as its own LSE partition and then
 * merged exactly: (A) keys that are not temporally biased guide keys, normal
 * logits; (B) the biased guide keys with every target row at -cap; (C) the
 * local correction e^s (e^-penalty - e^-cap) of target rows over guide keys
 * closer than the saturation gap window + falloff*sqrt(cap/strength). Each
 * pass visits only the key tiles holding keys of its term. N <= 2^20;
 * num_partitions and partition_bounds are ignored.
 * Two baselines, kept for comparison rather than use:
 * DENSE_BIAS: the bias of every (query, key) pair is first written to the
 * workspace as a dense fp32 tensor [B][N][npad] (npad = N rounded up to a
 * multiple of 64), and one fused pass then reads it instead of evaluating the
 * rule: the dense bias tensor that the "Three backends" section says the
 * Flash Partitions evaluation avoids building. TARA_BF16 only; the workspace
 * grows by 4*B*N*npad bytes (about 46 GB at N = 107,126).
 * FRAME_LOOP: the fused pass launched once per query range, in order on the
 * stream, each range against all keys: the per-frame attention loop that the
 * one-pass kernels of that section drop. The num_partitions ranges are given
 * by partition_bounds as query-row offsets (for instance one range per latent
 * frame of the target clip and one for the remaining rows), or are near-equal
 * when it is NULL; 1 <= num_partitions <= max(N, 1).
 * All modes return the same O and LSE up to rounding. */
typedef enum {
  TARA_MODE_FUSED = 0,
  TARA_MODE_PARTITIONED = 1,
  TARA_MODE_THREE_TERM = 2,
  TARA_MODE_DENSE_BIAS = 3,
  TARA_MODE_FRAME_LOOP = 4
} tara_mode_t;

typedef enum {
  TARA_OK = 0,
  TARA_ERR_NULL_POINTER = -1,       /* a required pointer is NULL */
  TARA_ERR_BAD_SHAPE = -2,          /* B, H or N negative or too large */
  TARA_ERR_UNSUPPORTED_DTYPE = -3,  /* dtype not TARA_BF16 / TARA_FP32 */
  TARA_ERR_UNSUPPORTED_HEAD_DIM = -4, /* D not 64 or 128 */
  TARA_ERR_BAD_STRIDE = -5,         /* base or stride not 16-byte aligned, or negative, or (bf16)
                                       too large for 32-bit tile offsets (see tara_attn_fwd) */
  TARA_ERR_BAD_PARAM = -6,          /* a control out of range (see tara_params_t) */
  TARA_ERR_WORKSPACE = -7,          /* workspace NULL or smaller than tara_workspace_bytes() */
  TARA_ERR_BAD_METADATA = -8,       /* only with TARA_VALIDATE=1: metadata out of range */
  TARA_ERR_HIP = -9                 /* a HIP runtime call failed (message in tara_last_error) */
} tara_status_t;

#define TARA_MAX_PICTURES 16
#define TARA_MAX_BINDINGS 4
#define TARA_MAX_PARTITIONS 64

/* Controls of one call. Start from tara_params_default().
 *  window, falloff, strength, cap: the four TARA controls ("The temporal rule";
 *    defaults 0.20 s, 0.25 s, 2.0, 6.0). Valid: finite, window >= 0,
 *    falloff > 0, strength >= 0, cap >= 0. strength == 0 or cap == 0 removes
 *    the temporal bias (plain attention on those edges).
 *  binding_enabled, num_pictures, num_bindings, picture_gain: reference
 *    binding ("Inputs you'll set": picture_index chooses the Picture whose
 *    gain is reference_strength, the other pictures get
 *    other_reference_strength; 1 is neutral). Here the gain is given per
 *    0-based picture id, 0 <= id < num_pictures <= TARA_MAX_PICTURES.
 *    num_bindings (1 .. TARA_MAX_BINDINGS; 0 is read as 1) bindings apply
 *    together, as chained binding nodes do ("Common issues": their log gains
 *    add): binding j uses picture_gain[j][*] and mask plane j. Every gain
 *    used must be finite and > 0. binding_enabled == 0 ignores picture_id,
 *    mask_weight and the gains.
 *  softmax_scale: multiplies Q . K only; 0 selects 1/sqrt(D).
 *  mode, num_partitions, partition_bounds: see tara_mode_t. partition_bounds
 *    is a host array of num_partitions + 1 non-decreasing offsets from 0 to N
 *    (key offsets in PARTITIONED mode, query-row offsets in FRAME_LOOP mode;
 *    empty ranges allowed), or NULL for num_partitions near-equal ranges;
 *    PARTITIONED: 1 <= num_partitions <= TARA_MAX_PARTITIONS.
 *  qk8: nonzero computes Q . K from 8-bit copies, as the dense 8-bit one-pass
 *    kernels of the "Three backends" section do (that section names no
 *    quantisation scheme; this one is): each query row and each tile of 64
 *    keys is divided by its own power of two, 2^(floor(log2 max|x|) - 7), and
 *    rounded to FP8 E4M3 (round to nearest even); the FP8 products are summed
 *    in fp32 and multiplied back by both powers of two. Softmax, bias and P.V
 *    are unchanged (P and V stay bf16). Requires TARA_BF16 and TARA_MODE_FUSED.
 *    The result equals exact attention on the rounded Q and K up to fp32
 *    rounding; against unrounded attention it differs by the E4M3 rounding of
 *    the logits (relative 2^-4 per element). */
typedef struct {
  float window;
  float falloff;
  float strength;
  float cap;
  int binding_enabled;
  int num_pictures;
  int num_bindings;
  float picture_gain[TARA_MAX_BINDINGS][TARA_MAX_PICTURES];
  float softmax_scale;
  int mode;
  int num_partitions;
  const int32_t* partition_bounds;
  int qk8;
} tara_params_t;

/* Fills *p with the defaults: window 0.20, falloff 0.25, strength 2.0,
 * cap 6.0, binding off (one binding, all gains 1), scale 1/sqrt(D), fused
 * mode. */
void tara_params_default(tara_params_t* p);

/* Device workspace tara_attn_fwd needs for this call shape (bytes, a multiple
 * of 256). It holds per-token encodings of the metadata (with binding, a
 * per-query table of the summed log gains of every picture), per-key-tile
 * summaries, V laid out key-contiguous per (batch, head, dim) for the bf16
 * path, per-partition O/LSE in the partitioned and three-term modes, the FP8
 * keys with qk8 and the dense bias in DENSE_BIAS mode. Returns 0 for an empty
 * call (B, H or N == 0) and (size_t)-1 for arguments tara_attn_fwd would reject
 * (p == NULL, bad dtype or head dim, bad partition count, qk8 outside bf16
 * fused mode, DENSE_BIAS with fp32). */
size_t tara_workspace_bytes(int dtype, int B, int H, int N, int D,
                            const tara_params_t* p);

/* TARA-biased attention forward: O = softmax(logits) V and LSE per query row.
 *
 *  q, k, v  device, dtype elements, logical shape [B][H][N][D], element
 *           (b,h,n,d) at base + b*str[0] + h*str[1] + n*str[2] + d (d contiguous).
 *           Base addresses 16-byte aligned; every stride a multiple of
 *           16 bytes / sizeof(element) and >= 0. bf16: the kernel addresses
 *           one head's key rows with 32-bit byte offsets, so k_str[2] * 2 *
 *           Npad and D * Npad * 2 (Npad: N rounded up to 64) must be < 2^31
 *           (else TARA_ERR_BAD_STRIDE).
 *  o        device, same dtype and layout rules (strides o_str); fully written.
 *  lse      device fp32 [B][H][N] contiguous, natural log; fully written.
 *  dtype    a tara_dtype_t value: TARA_BF16 (bf16 in and out, fp32
 *           accumulation) or TARA_FP32; any other int is rejected (the
 *           parameter is an int so that every value a caller may pass is
 *           well defined).
 *  D        64 or 128.
 *  seg_type device uint8 [B][N], TARA_SEG_* codes.
 *  token_time device fp32 [B][N], seconds on the aligned output clock; read
 *           only for TARGET and GUIDE tokens (others may hold anything).
 *  picture_id device int16 [B][N], 0-based picture id of PICTURE tokens; read
 *           only when binding is active; may be NULL when it is not.
 *  mask_weight device fp32 [num_bindings][B][N] mask weight m of TARGET
 *           queries, one plane per binding, or NULL for m = 1 on every target
 *           query ("BFS H3 Reference Attention Binding (Experimental)",
 *           section "Inputs you'll set"). Read only when binding is active.
 *  p        host, the controls (see tara_params_t).
 *  workspace device, >= tara_workspace_bytes(...) bytes, 256-byte aligned;
 *           contents on entry are ignored, on exit unspecified.
 *  stream   HIP stream the work is enqueued on.
 *
 * Metadata out of range is not an error by default and never causes an
 * out-of-bounds read; the token loses only the term its bad field feeds:
 * seg_type > 3 makes it an OTHER token, a picture id outside [0, num_pictures)
 * removes its binding term, a non-finite time takes a GUIDE key or a TARGET
 * query out of the temporal term (the query keeps its binding term), and a
 * non-finite mask weight removes that binding's term for its query. With the environment
 * variable TARA_VALIDATE=1 the metadata is copied to the host and checked
 * first (synchronously), returning TARA_ERR_BAD_METADATA.
 * B, H or N == 0 is a valid empty call and enqueues nothing. */
int tara_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int dtype, int B, int H, int N, int D,
                  const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
                  const int64_t o_str[3],
                  const uint8_t* seg_type, const float* token_time,
                  const int16_t* picture_id, const float* mask_weight,
                  const tara_params_t* p, void* workspace, size_t workspace_bytes,
                  tara_stream_t stream);

/* Workspace of tara_attn_fwd_noalloc, in bytes: a fixed device array of the
 * library (128 MiB on each device it runs on, held until the process ends). */
#define TARA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* tara_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, rules and results as tara_attn_fwd, without the workspace:
 * the library's own device array of TARA_NOALLOC_SCRATCH_BYTES serves as the
 * workspace, and the call is worked through one batch element and as many
 * heads as that array holds at a time, in order on `stream`, with the same
 * kernels. Allocates nothing (no hipMalloc, no host allocation on the call
 * path). The first call on a device looks the array's device address up once.
 * Every call on one device shares that device's array and leaves its last
 * contents there (nothing in it has to start at zero): calls that overlap on
 * one device (on different streams, or from threads not ordered on one
 * stream) race and give wrong results; calls in order on one stream do not.
 * Errors: as tara_attn_fwd, plus TARA_ERR_WORKSPACE when one head of one batch
 * element needs more workspace than the array holds (for instance the
 * DENSE_BIAS baseline beyond about 5,000 tokens). This entry point does not
 * record timing events and ignores TARA_VALIDATE and the tile-class readback,
 * which synchronise or allocate. */
int tara_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int dtype, int B, int H, int N, int D,
                          const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
                          const int64_t o_str[3],
                          const uint8_t* seg_type, const float* token_time,
                          const int16_t* picture_id, const float* mask_weight,
                          const tara_params_t* p, tara_stream_t stream);

/* Static English text for a status code (never NULL). */
const char* tara_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). The pointer
 * stays valid until this thread's next tara_* call. */
const char* tara_last_error(void);

/* What the last successful tara_attn_fwd on this thread ran.
 *
 * Tile classes (debug readback). The bf16 kernel applies the bias per key tile
 * of 64 keys and per wave of 32 query rows: for each row a constant over the
 * tile (plain: no bias; saturated: a guide tile entirely past the saturation
 * gap window + falloff*sqrt(cap/strength), every logit -cap; window: a guide
 * tile entirely inside the free window; picture: a tile of one bound
 * picture's keys, the row's summed log gain), or the per-element formula when
 * some row of the wave needs it (elem: mixed tiles, guide tiles straddling a
 * knot, partition edges, or every tile under TARA_DISABLE_TILE_SKIP=1). With
 * the environment variable TARA_TILE_STATS=1 (or TARA_LOG=1), a bf16 call in
 * FUSED or PARTITIONED mode replays that decision for every (query row, key
 * tile) pair in a debug kernel, waits for the stream and fills the tiles_*
 * counts, summed over batch elements and heads (so they add up to
 * B * H * N * the number of key tiles visited); tile_stats is then 1.
 * Otherwise tile_stats is 0 and the counts are 0. */
typedef struct {
  int mode;              /* tara_mode_t */
  int dtype;             /* tara_dtype_t */
  int bias_active;       /* strength > 0 and cap > 0 */
  int binding_active;    /* binding_enabled and some gain != 1 */
  int num_partitions;    /* 1 in fused mode; query ranges in FRAME_LOOP mode */
  int block_q;           /* query rows per workgroup of the attention kernel */
  int block_k;           /* keys per tile */
  int grid;              /* workgroups of the attention kernel (all partitions and passes) */
  int launches;          /* kernels enqueued by the call (the debug kernel not counted) */
  int elem_all;          /* 1 when TARA_DISABLE_TILE_SKIP=1 sent every tile down the per-element path */
  int tile_stats;        /* 1 when the counts below were taken */
  int tail_parts;        /* fused bf16: key ranges of the range pass that took the last query blocks
                            of every (batch, head) (their workgroups would have left the last round
                            of compute units partly filled); 0 when the fused pass took all rows */
  long long tiles_plain, tiles_saturated, tiles_window, tiles_picture, tiles_elem;
} tara_run_info_t;

/* Copies the run info of this thread's last successful call; TARA_ERR_NULL_POINTER
 * if info is NULL. */
int tara_get_last_run_info(tara_run_info_t* info);

/* Per-launch timing of the attention kernel, for measurement. With timing on,
 * every tara_attn_fwd records a HIP event pair on its stream around the
 * attention kernel (the partition merge is not included). tara_timing_read
 * waits for the recorded pairs, writes up to `max` durations in milliseconds
 * to ms_out (host), sets *count to how many were written, and forgets all
 * recorded pairs. Global to the process (not per thread). */
int tara_timing_enable(int on);
int tara_timing_read(float* ms_out, int max, int* count);

/* Operand kinds of tara_probe_mfma_bf16. */
typedef enum {
  TARA_PROBE_CONSTANT = 0, /* every product on the same two fragments: few bits
                              toggle and the clock stays near its top, so this
                              is the rate at which the matrix cores issue */
  TARA_PROBE_RANDOM = 1    /* each wave cycles through 8 + 8 fragments of
                              varied bf16 values, as real data does: the power
                              limit sets the clock, so this is the practical
                              ceiling for MFMA work on real data */
} tara_probe_operands_t;

/* Measurement aid, not part of the attention path: runs a kernel made only of
 * back-to-back bf16 MFMAs (v_mfma_f32_32x32x16_bf16) on register operands of
 * the given kind (a tara_probe_operands_t), two waves per SIMD on every CU,
 * `iterations` rounds of four products per wave, on `stream` of the current
 * device (one untimed launch, then one timed with HIP events), and stores the
 * rate in *tflops. Those rates are the MFMA ceilings the attention kernel
 * meets on this device, beside the nominal dense bf16 peak. Blocks until the
 * launch completes. Returns TARA_ERR_NULL_POINTER for a NULL tflops,
 * TARA_ERR_BAD_PARAM unless 1 <= iterations <= 2^24 and `operands` is one of
 * the kinds (checked before any device work), TARA_ERR_HIP if a HIP call
 * fails. */
int tara_probe_mfma_bf16(int iterations, int operands, float* tflops, tara_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TARA_H_ */
