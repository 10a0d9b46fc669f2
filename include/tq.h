/*
 * tq.h - C ABI of the TurboQuant KV-cache library for AMD MI355X (gfx950).
 *
 * What the library computes (page titles and sections of the TurboQuant pages):
 *   "TurboQuant QJL投影深度剖析" (QJL deep-dive), section 2: a key x is stored as
 *   ||x||, the (b-1)-bit Lloyd-Max codes of the rotated unit vector Pi x/||x||,
 *   the signs of S r for the residual r = x - x~ (d bits in d/8 bytes) and ||r||.
 *   Section 5: the record is (codes, sign bytes, ||r||, ||x||), bit-packed, and
 *   <q, x~> + ||r|| sqrt(pi/2)/d <S q, signs> estimates <q, x> without bias.
 *   Section 6: scores use the forward-rotated query Pi q against the centroids
 *   and the pre-sketched query S q against the signs; decode attention runs an
 *   online softmax over the whole packed cache in one pass; each layer seeds
 *   its own Pi/S with 42 + 7 * layer.
 *   "TurboQuant MLX port" write-up (cf-1.com), 背景: values use the MSE-only
 *   path (codes + ||v||); 直接构造缓存: key_bits = 0 keeps K in fp16.
 *
 * Conventions shared by every call
 *   - d (head_dim) is 128 for the device calls.
 *   - All device pointers are plain device (HBM) addresses owned by the
 *     caller; the library never allocates, frees or retains device memory and
 *     keeps no mutable global state (apart from the per-thread error message,
 *     the per-device address of tq_decode_attention_noalloc's static scratch
 *     and the test hook tq_set_append_wait), so calls on different streams
 *     may run concurrently.  `stream` is a hipStream_t (NULL = the default
 *     stream).
 *   - Device calls validate their host-side arguments synchronously and
 *     return a status; kernels are then enqueued on `stream` and never trap.
 *     TQ_ERR_HIP reports a failed launch.  tq_last_error() gives a
 *     thread-local message for the last failing call.  No C++ exception
 *     crosses this boundary.
 *   - NaN inputs propagate to the affected norms and outputs; a zero vector
 *     compresses to zero norms and contributes nothing.
 *
 * Packed cache layout (one set of planes for n_layers layers, each plane laid
 * out [layer][kv_head][...]; capacity is a multiple of 32 slots):
 *   k_idx   uint8  [L][H][capacity][d*(k_bits-1)/8]  LSB-first codes, coord j at
 *                                                      bits [j*m, (j+1)*m), m = k_bits-1
 *   k_sign  uint8  [L][H][capacity][d/8]             bit j = (S r)_j >= 0
 *   k_norm  float  [L][H][capacity]                  ||x||
 *   k_rnorm float  [L][H][capacity]                  ||r||
 *   k_f16   half   [L][H][capacity][d]               keys kept in fp16 (k_bits = 0)
 *   v_idx   uint8  [L][H][capacity/32][d][4*v_bits]  per 32-slot block and coord j,
 *                                                      slot p of the block at bits
 *                                                      [p*v_bits, (p+1)*v_bits)
 *   v_norm  float  [L][H][capacity]                  ||v||
 *   v_f16   half   [L][H][capacity/32][d][32]        values kept in fp16 (v_bits = 0)
 * Planes that a format does not use may be NULL.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tq_status;
enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad layout */
  TQ_ERR_UNSUPPORTED = 2, /* d != 128 on device, bit width out of range */
  TQ_ERR_WORKSPACE = 3,   /* workspace too small */
  TQ_ERR_HIP = 4,         /* a HIP launch failed */
  TQ_ERR_APPEND_TIMEOUT = 5 /* tq_decode_step_check: a decode wave stopped waiting for the step's append */
};

enum { TQ_DTYPE_F32 = 0, TQ_DTYPE_BF16 = 1, TQ_DTYPE_F16 = 2 };

/* Storage format.  k_bits: 0 keeps keys in fp16, else 2..5 or 8 total bits
 * per coordinate = (k_bits-1) Lloyd-Max bits + 1 QJL sign bit (8: the 8-bit
 * key codec, turbo8, of the long-context write-up's benchmarks).  v_bits: 0
 * keeps values in fp16, else 1 to 4 MSE-only bits. */
typedef struct tq_format {
  int32_t d;
  int32_t k_bits;
  int32_t v_bits;
} tq_format;

/* Per-layer tables in device memory (fp32).  pi, s and pi_s hold n_layers
 * consecutive row-major d x d matrices (layer l at offset l*d*d): the rotation
 * Pi (y = Pi x), the QJL sketch S and their product M = S Pi^T, as written by
 * tq_make_rotations.  Codebooks are shared by all layers: 2^m ascending
 * centroids and 2^m - 1 boundaries for the key (m = k_bits-1) and value
 * (m = v_bits) quantisers, as written by tq_make_codebook (rounded to fp32).
 * Compression compares rotated coordinates with the fp32 boundaries and forms
 * the key residual with the fp32 centroids.  Decode feeds the centroids to
 * fp16 MFMA operands: keys of 3 or more Lloyd-Max bits as an fp16 high part
 * and remainder (about 22 significant bits); keys of 1 or 2 Lloyd-Max bits and
 * all values as one fp16 value per centroid of the codebook scaled by
 * k_operand_scale / v_operand_scale, numbers in [1, 2) that the caller takes
 * from tq_fp16_operand_scale (host) for the same fp32 centroids; a value
 * outside [1, 2) (e.g. 0) means 1, plain fp16 rounding, which on sharp
 * softmaxes can move outputs by more than 1e-3. */
typedef struct tq_tables {
  const float* pi;
  const float* s;
  const float* pi_s;
  const float* k_centroids;
  const float* k_boundaries;
  const float* v_centroids;
  const float* v_boundaries;
  float k_operand_scale;
  float v_operand_scale;
} tq_tables;

/* Device planes of a packed cache (layout above). */
typedef struct tq_cache {
  int32_t n_layers;
  int32_t n_kv_heads;
  int64_t capacity;
  uint8_t* k_idx;
  uint8_t* k_sign;
  float* k_norm;
  float* k_rnorm;
  void* k_f16;
  uint8_t* v_idx;
  float* v_norm;
  void* v_f16;
} tq_cache;

/* Seed of a layer's Pi/S stream: 42 + 7 * layer (QJL deep-dive, section 6). */
uint64_t tq_layer_seed(int32_t layer);

/* Host.  Builds Pi (Haar orthogonal: Q * diag(sign R_ii) of the Householder
 * QR of a d x d matrix of normals 0..d*d-1) and S (normals d*d..2*d*d-1), both
 * from the SplitMix64 + Box-Muller stream of `seed` (QJL deep-dive, section 2
 * steps 1 and 3), and optionally M = S Pi^T, computed in double from the fp32
 * Pi and S.  Outputs are fp32 row-major d x d in caller-owned host memory;
 * pi_s may be NULL.  3 <= d <= 1024.  Deterministic. */
tq_status tq_make_rotations(int32_t d, uint64_t seed, float* pi, float* s, float* pi_s);

/* Host.  Lloyd-Max quantiser (QJL deep-dive, section 2 step 2) for one
 * coordinate of a uniformly random unit vector in R^d, density
 * Gamma(d/2)/(sqrt(pi) Gamma((d-1)/2)) (1-t^2)^((d-3)/2) on [-1, 1].
 * Writes 2^bits ascending centroids and 2^bits - 1 boundaries (midpoints) in
 * double to caller-owned host arrays.  1 <= bits <= 8, 3 <= d <= 65536. */
tq_status tq_make_codebook(int32_t d, int32_t bits, double* centroids, double* boundaries);

/* Host.  The scale alpha in [1, 2) of a codebook's fp16 decode operands: the
 * one, among the alphas that put some centroid magnitude exactly on an fp16
 * value, for which the largest relative rounding error of fp16(alpha |c_k|)
 * over the nonzero magnitudes is smallest (ties: the smallest such alpha).
 * An fp16 operand keeps 11 significant bits, so a centroid rounded to fp16 is
 * off by up to 2^-12 of its value; scaled, a codebook with one or two
 * magnitudes is exact to about 2^-20 and the 16-level one to about 2^-13.5.
 * centroids: n fp32 values in host memory (1 <= n <= 256).  Returns 1 for
 * invalid input or a codebook without a nonzero finite magnitude. */
float tq_fp16_operand_scale(const float* centroids, int32_t n);

/* Byte sizes of the eight cache planes for a format, in the order
 * k_idx, k_sign, k_norm, k_rnorm, k_f16, v_idx, v_norm, v_f16 (0 = unused). */
tq_status tq_cache_plane_bytes(const tq_format* fmt, int32_t n_layers, int32_t n_kv_heads,
                               int64_t capacity, size_t out_bytes[8]);

/* Workspace bytes tq_decode_attention and tq_score need for these sizes
 * (0 on invalid input). */
size_t tq_decode_workspace_bytes(const tq_format* fmt, int32_t n_layers, int32_t batch,
                                 int32_t n_kv_heads, int32_t n_q_heads, int64_t max_seq_len);

/* Host.  The work split of a decode / score call for these sizes:
 * out[0] problems (layer x sequence x KV head x group of <= 8 query heads),
 * out[1] 32-token chunks per problem (from max_seq_len, possibly padded with
 * chunks that hold no tokens), out[2] chunks per decode workgroup,
 * out[3] decode workgroups, out[4] pieces per problem at most.  Workgroup w
 * takes chunks [w out[2], (w + 1) out[2]) of the problem-major chunk sequence
 * (the last run shorter).  TQ_ERR_INVALID_ARG on invalid sizes. */
tq_status tq_decode_split(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                          int32_t n_q_heads, int64_t max_seq_len, int64_t out[5]);

/* Device.  Compresses keys and values and writes them into the cache
 * (QJL deep-dive, section 2; MLX write-up, 背景).  k and v are device arrays
 * [n_layers][n_tokens][n_kv_heads][d] of `dtype` (TQ_DTYPE_F32/BF16/F16) for
 * cache layers layer0 .. layer0+n_layers-1.  Token i goes to slot
 * slots[i] (device int64 array, same for every layer) or, when slots is
 * NULL, to slot0 + i.  Slots must be distinct within one call and lie in
 * [0, capacity); out-of-range slots are skipped by the kernel.  Records of
 * other slots are left untouched.  Enqueued on `stream`. */
tq_status tq_compress_kv(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                         const void* k, const void* v, int32_t dtype, int32_t layer0,
                         int32_t n_layers, int64_t n_tokens, const int64_t* slots, int64_t slot0,
                         void* stream);

/* Device.  tq_compress_kv with the bulk kernel (16 or more tokens) held to at
 * most max_workgroups workgroups, hence CUs (0 means no bound; fewer tokens
 * use the append kernel as in tq_compress_kv).  For compression that runs in
 * the background on a second stream while decode calls run on another: the
 * decode kernel of a call uses tq_decode_split(...)'s n_workgroups CUs, so a
 * bound of 256 minus that count leaves it its CUs (the MLX write-up, section
 * on the delegated cache, recompresses its packed store in the background).
 * Records are the same as tq_compress_kv's, bit for bit.  Arguments,
 * layouts, ownership and errors as tq_compress_kv; max_workgroups < 0 is
 * TQ_ERR_INVALID_ARG. */
tq_status tq_compress_kv_bounded(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                 const void* k, const void* v, int32_t dtype, int32_t layer0, int32_t n_layers,
                                 int64_t n_tokens, const int64_t* slots, int64_t slot0, int32_t max_workgroups,
                                 void* stream);

/* Device.  Single-query decode attention over the packed cache for every
 * layer of the cache (QJL deep-dive, sections 5 and 6): for query head h
 * (KV head h / (n_q_heads / n_kv_heads)), logits
 *   l_t = scale * (||x_t|| <Pi q, c[idx_t]> + ||r_t|| sqrt(pi/2)/d <S q, 2 s_t - 1>)
 * (scale * <q, k_t> for fp16 keys), softmax over the sequence's tokens and
 * out = sum_t p_t v~_t with v~_t = ||v_t|| Pi^T c_v[idx_t] (fp16 values as
 * stored).  q and out are device float [n_layers][batch][n_q_heads][d].
 * seq_start (int64) and seq_len (int32) are device arrays [batch]: sequence
 * b occupies slots [seq_start[b], seq_start[b] + seq_len[b]); seq_start must
 * be a multiple of 32; the kernels clamp a sequence to the capacity and to max_seq_len and treat
 * a misaligned or negative start as empty.  An empty sequence gives a zero
 * output row.  max_seq_len (host) bounds every seq_len and sizes the work
 * decomposition.  scale = 0 means 1/sqrt(d).  n_q_heads must be a multiple of
 * n_kv_heads.  workspace: device scratch of at least
 * tq_decode_workspace_bytes(...) bytes; enqueued on `stream`. */
tq_status tq_decode_attention(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                              const float* q, int32_t batch, int32_t n_q_heads,
                              const int64_t* seq_start, const int32_t* seq_len,
                              int64_t max_seq_len, float scale, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Device.  Decode attention over sequences held in two parts: the older
 * tokens packed in `cache` and the most recent ones kept at full (fp16)
 * precision in `tail`, a cache of the fp16 format (k_bits = v_bits = 0, same
 * d, n_layers and n_kv_heads), with one softmax over both (the MLX write-up,
 * sections on building the cache and on limits, and the QJL deep-dive,
 * section 6: recent tokens stay uncompressed).  Sequence b holds packed slots
 * [seq_start[b], + seq_len[b]) of `cache` and tail slots [tail_start[b],
 * + tail_len[b]) of `tail`; both parts follow tq_decode_attention's rules
 * (starts a multiple of 32, lengths clamped to the capacity and to
 * max_seq_len / max_tail_len, misaligned or negative starts empty).  q, out,
 * scale and the head mapping as in tq_decode_attention.  Tokens enter the
 * tail with tq_compress_kv on the fp16 format (the values stored as fp16),
 * and move to the packed cache with tq_compress_kv from those fp16 values.
 * workspace: at least tq_decode_tail_workspace_bytes(...) bytes; it holds the
 * packed decode's piece counters (zeroed by the call's own query
 * preparation), so calls on one workspace must not overlap. */
tq_status tq_decode_attention_tail(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                   const tq_cache* tail, const float* q, int32_t batch, int32_t n_q_heads,
                                   const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                                   const int64_t* tail_start, const int32_t* tail_len, int64_t max_tail_len,
                                   float scale, float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Device, measurement only.  Reads `bytes` (a multiple of 16) of device
 * memory at `data` once, as a plain streaming read by n_workgroups workgroups
 * of 256 threads, and adds one sum per workgroup into partial[n_workgroups]
 * (device float, caller-zeroed): the reference for the achievable HBM read
 * bandwidth against which the decode kernel's rate can also be read. */
tq_status tq_stream_read_probe(const void* data, size_t bytes, float* partial, int32_t n_workgroups, void* stream);

/* The recent-token ring of a hybrid cache (packed history + fp16 tail).
 * The pages keep the most recent tokens at full precision in a ring buffer,
 * take the compressed path only once there is history enough (16 tokens or
 * more: the QJL deep-dive, section 6), and compress only sequences of at
 * least min_compress_tokens tokens (default 256: the MLX write-up, section on
 * the quality scripts).  Convention here: a ring of ring_cap slots (a
 * multiple of 32) lives in a tail cache of the fp16 format with capacity >=
 * 2 ring_cap, every token stored at its ring slot p and again at p +
 * ring_cap, so that any run of at most ring_cap consecutive ring positions
 * starting at p < ring_cap is the contiguous slot range [p, p + n) of the
 * tail; a sequence's tail is then one range for tq_decode_attention_tail even
 * when it wraps around the ring.  Tokens leave the ring, oldest first, in
 * whole 32-token blocks (tq_tail_policy), so ring heads stay multiples of 32
 * and the packed part of a sequence, once non-empty, holds 32 tokens or more.
 *
 * Host.  Per sequence b (host arrays of `batch`): n_flush[b] = the largest
 * multiple of 32 that leaves at least keep_recent tokens in the tail, when
 * packed_len[b] + tail_len[b] >= min_compress_tokens, else 0.
 * TQ_ERR_INVALID_ARG for negative lengths or parameters or NULL arrays. */
tq_status tq_tail_policy(int32_t batch, const int32_t* packed_len, const int32_t* tail_len,
                         int32_t min_compress_tokens, int32_t keep_recent, int32_t* n_flush);

/* Device.  Writes n_tokens new tokens into the ring of `tail` (fp16 format
 * with d = fmt->d): token i (k, v as in tq_compress_kv, [n_layers][n_tokens]
 * [H][d]) at tail slots ring_slots[i] and ring_slots[i] + ring_cap (device
 * int64 [n_tokens], each in [0, ring_cap)).  Two compression launches on
 * `stream`.  TQ_ERR_INVALID_ARG unless ring_cap is a positive multiple of 32
 * with 2 ring_cap <= tail->capacity. */
tq_status tq_tail_append(const tq_format* fmt, const tq_tables* tables, const tq_cache* tail, const void* k,
                         const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                         const int64_t* ring_slots, int64_t ring_cap, void* stream);

/* Host.  Workspace bytes of tq_tail_flush (0 for invalid sizes). */
size_t tq_tail_flush_workspace_bytes(const tq_format* fmt, const tq_cache* packed, int32_t batch, int32_t max_flush);

/* Device.  Moves tail tokens into the packed cache: for every layer of the
 * caches, token i < n_flush[b] of sequence b (tail slot tail_pos[b] + i) is
 * compressed from its fp16 key and value into packed slot dst_slot[b] + i
 * (device arrays of `batch`: int64 tail_pos, int32 n_flush (each <=
 * max_flush), int64 dst_slot).  The tail is not modified (the caller advances
 * its ring head).  A gather launch into the workspace (fp16 staging of
 * batch x max_flush tokens, then their packed slots), then the compression;
 * tokens whose tail or packed slot is outside its cache are skipped.
 * workspace: at least tq_tail_flush_workspace_bytes(fmt, packed, batch,
 * max_flush) bytes, not shared by overlapping calls. */
tq_status tq_tail_flush(const tq_format* fmt, const tq_tables* tables, const tq_cache* packed, const tq_cache* tail,
                        int32_t batch, int32_t max_flush, const int64_t* tail_pos, const int32_t* n_flush,
                        const int64_t* dst_slot, void* workspace, size_t workspace_bytes, void* stream);

/* Host.  Workspace bytes of tq_decode_attention_tail (0 for invalid sizes). */
size_t tq_decode_tail_workspace_bytes(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                                      int32_t n_q_heads, int64_t max_seq_len, int64_t max_tail_len);

/* Device.  tq_decode_attention in three stages, for callers that schedule
 * them separately (and for timing the kernels one by one).  They take the same
 * arguments as tq_decode_attention and share its workspace, which carries the
 * prepared queries and the partial results from one stage to the
 * next:
 *   tq_decode_prepare  - forward-rotated and pre-sketched queries Pi q, S q
 *                        (QJL deep-dive, section 6: sketched once per query);
 *   tq_decode_partials - scores every token of every (layer, sequence, KV
 *                        head) on the packed cache and accumulates the
 *                        softmax-weighted values (online softmax) in pieces of
 *                        equal size, one partial result per piece and head;
 *   tq_decode_combine  - merges the pieces of each query head and applies Pi^T.
 * Calling them in this order on one stream gives tq_decode_attention's result.
 * The decode kernel deals token chunks to its waves dynamically, so any two
 * calls (staged or not) may differ in the last bits.  The max_seq_len / batch
 * / head arguments must be the same in all three calls. */
tq_status tq_decode_prepare(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const float* q,
                            int32_t batch, int32_t n_q_heads, int64_t max_seq_len, void* workspace,
                            size_t workspace_bytes, void* stream);

tq_status tq_decode_partials(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                             int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len,
                             int64_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                             void* stream);
tq_status tq_decode_combine(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                            int32_t n_q_heads, int64_t max_seq_len, float* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Device.  tq_decode_partials and tq_decode_combine in one launch (the
 * attention of the QJL deep-dive, section 6, on queries already prepared by
 * tq_decode_prepare or tq_append_prepare on the same workspace): each
 * problem's pieces are merged by the workgroup that writes its last piece, so
 * out is written by the decode kernel itself.  Same arguments, layouts and
 * errors as those two calls; out as in tq_decode_attention.  The workspace
 * holds one piece counter per problem: the preparation sets them to zero and
 * every completed call leaves them at zero, so two calls on one workspace
 * must not overlap. */
tq_status tq_decode_attend(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                           int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                           float scale, float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Device.  A decode step's append and query preparation in one launch: the
 * same result as tq_compress_kv(fmt, tables, cache, k, v, dtype, layer0,
 * n_layers, n_tokens, slots, slot0, stream) followed by
 * tq_decode_prepare(fmt, tables, cache, q, batch, n_q_heads, max_seq_len,
 * workspace, workspace_bytes, stream), with their arguments, layouts,
 * ownership and errors; both are checked before anything is enqueued.  The
 * new tokens' records (QJL deep-dive, sections 2 and 5) and the sketched
 * queries (section 6) do not depend on each other, so for fewer than 16
 * tokens one kernel computes both; for 16 or more tokens the two calls are
 * made one after the other.  Follow it with tq_decode_attend (or
 * tq_decode_partials and tq_decode_combine) on the same workspace. */
tq_status tq_append_prepare(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                            const void* k, const void* v, int32_t dtype, int32_t layer0, int32_t n_layers,
                            int64_t n_tokens, const int64_t* slots, int64_t slot0, const float* q, int32_t batch,
                            int32_t n_q_heads, int64_t max_seq_len, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Device.  A whole decode step: tq_compress_kv(fmt, tables, cache, k, v,
 * dtype, layer0, n_layers, n_tokens, slots, slot0, stream) followed by
 * tq_decode_attention(fmt, tables, cache, q, batch, n_q_heads, seq_start,
 * seq_len, max_seq_len, scale, out, workspace, workspace_bytes, stream), with
 * their arguments, layouts, ownership and errors; both are checked before
 * anything is enqueued.  When the append takes at most 32 workgroups (one
 * per 8 (token, KV head) items per layer) it takes two launches: the query
 * preparation, then the decode kernel, whose first workgroups compress the
 * new tokens (QJL deep-dive, sections 2 and 5) while the others start the
 * attention (section 6) on the CUs the append leaves; a decode wave waits for
 * its layer's append only before it reads a chunk that may hold a new token
 * (slots [slot0, slot0 + n_tokens) of each appended plane, or any slot when
 * `slots` is given).  Larger appends run before the decode: in the query
 * preparation's launch for fewer than 16 tokens (tq_append_prepare, then
 * tq_decode_attend), else as tq_compress_kv then tq_decode_attention.  The
 * workspace is tq_decode_attention's; calls on one workspace must not
 * overlap. */
tq_status tq_decode_step(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const void* k,
                         const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                         const int64_t* slots, int64_t slot0, const float* q, int32_t batch, int32_t n_q_heads,
                         const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

/* One part of a decode step over a model whose layers use different formats
 * (tq_decode_step_parts): the arguments of tq_decode_step that belong to the
 * part, with their meaning there.  k, v: the new tokens of cache layers
 * [layer0, layer0 + n_layers) of this part's cache, laid out as for
 * tq_compress_kv; q, out: [cache->n_layers][batch][n_q_heads][d] fp32;
 * workspace: at least tq_decode_workspace_bytes for this part's cache. */
typedef struct tq_step_part {
  const tq_format* fmt;
  const tq_tables* tables;
  const tq_cache* cache;
  const void* k;
  const void* v;
  int32_t layer0;
  int32_t n_layers;
  const float* q;
  float* out;
  void* workspace;
  size_t workspace_bytes;
} tq_step_part;

/* Device.  A decode step over n_parts caches of different formats that share
 * the batch, its sequences and the new tokens' slots (say a model that keeps
 * its first and last two KV layers in fp16 and its other layers with fp16
 * keys and quantized values: the asymmetric mode with boundary-layer
 * protection of the TurboQuant Apple-MLX port write-up, section on symmetric
 * and asymmetric compression): the same result as tq_decode_step for parts[0], then
 * parts[1], ..., each with its part's arguments and the shared ones given
 * here (dtype, n_tokens, slots, slot0, batch, n_q_heads, seq_start, seq_len,
 * max_seq_len, scale), with their layouts, ownership and errors.  Every part
 * is checked before anything is enqueued.  With two parts, the second with
 * fp16 keys and values (k_bits = v_bits = 0), and both appends small enough to
 * run inside the decode launch (at most 32 append workgroups in all), the two
 * decodes run in one launch: the decode workgroups are shared between the
 * parts in proportion to an estimate of each part's work per token (the bytes
 * it reads plus a fixed cost per token), so the launch pays one start and one
 * end instead of two.  Otherwise the parts' tq_decode_step
 * calls are made one after the other.  n_parts: 1 to 8; parts must not be
 * NULL; calls on one workspace must not overlap. */
tq_status tq_decode_step_parts(const tq_step_part* parts, int32_t n_parts, int32_t dtype, int64_t n_tokens,
                               const int64_t* slots, int64_t slot0, int32_t batch, int32_t n_q_heads,
                               const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                               void* stream);

/* Device.  The decode of tq_decode_step_parts alone, on queries already
 * prepared in each part's workspace (tq_decode_prepare or tq_append_prepare
 * for each part): the same result as tq_decode_attend for parts[0], then
 * parts[1], ..., with the shared arguments given here, their layouts,
 * ownership and errors, and two parts in one launch on the same condition as
 * tq_decode_step_parts (no append here).  The parts' k, v, layer0 and n_layers
 * are not read. */
tq_status tq_decode_attend_parts(const tq_step_part* parts, int32_t n_parts, int32_t batch, int32_t n_q_heads,
                                 const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                                 void* stream);

/* Host, synchronous.  Whether the last tq_decode_step on `workspace` (made
 * with these sizes) ran its append inside the decode launch without a decode
 * wave giving up its wait.  A wave that must read a chunk holding a new token
 * waits for the layer's append workgroups with a bounded wait (about a
 * second); if the wait ends unmet it records that in a flag word of the
 * workspace (zeroed by every call's query preparation) and reads the chunk
 * anyway, which may then miss the new tokens.  Synchronizes `stream`, reads
 * the flag; TQ_OK if clear, TQ_ERR_APPEND_TIMEOUT if set, TQ_ERR_WORKSPACE /
 * TQ_ERR_INVALID_ARG for bad arguments, TQ_ERR_HIP if the read fails. */
tq_status tq_decode_step_check(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                               int32_t n_q_heads, int64_t max_seq_len, const void* workspace, size_t workspace_bytes,
                               void* stream);

/* Host, test hook.  Sets the bounded wait of later tq_decode_step launches:
 * at most max_polls polls of the append count (default 1 << 20), waiting for
 * extra_groups more append workgroups than the launch has (default 0: any
 * other value makes the wait unmeetable, for testing the give-up path).
 * Process-wide; not for concurrent use with decode calls.  max_polls = 0 or
 * extra_groups < 0 is TQ_ERR_INVALID_ARG. */
tq_status tq_set_append_wait(uint32_t max_polls, int32_t extra_groups);

/* Device.  The scoring half of tq_decode_attention alone (the pages' separate
 * MSE-score and QJL-score kernels, QJL deep-dive section 6): writes the
 * logits l_t defined above to logits[n_layers][batch][n_q_heads][max_seq_len]
 * (device float; entries at t >= seq_len[b] are left untouched).  Same
 * arguments and workspace as tq_decode_attention.
 *
 * Several queries per sequence (a prefill chunk scored against the cache):
 * pass n_q query rows per head as n_q_heads * n_q heads, query j of head h at
 * index h * n_q + j (q viewed as [n_layers][batch][n_q_heads][n_q][d]); head
 * index / (n_q_heads * n_q / n_kv_heads) is still the KV head, so the logits
 * (and tq_decode_attention's outputs) come out as [..][n_q_heads][n_q][..].
 * The kernels take up to 8 such rows per pass over a KV head's codes. */
tq_status tq_score(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                   const float* q, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                   const int32_t* seq_len, int64_t max_seq_len, float scale, float* logits,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Device.  tq_score for many query rows per KV head (a prefill chunk's
 * queries against the compressed cache: the pages' separate MSE-score and
 * QJL-score kernels, QJL deep-dive section 6, with the query rows as the
 * columns of one contraction).  Same arguments, logits and workspace as
 * tq_score; query rows are heads, n_q_heads / n_kv_heads (G) of them per KV
 * head, e.g. 8 heads x 8 query tokens.  Where tq_score's kernel reads and
 * decodes a KV head's codes once per 8 rows, this one does once per 64 rows
 * (rows 64 g .. 64 g + 63 of a KV head per pass), its scores on fp16 MFMA
 * with the same operand precision. */
tq_status tq_score_multi(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const float* q,
                         int32_t batch, int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len,
                         int64_t max_seq_len, float scale, float* logits, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of the static device scratch of tq_decode_attention_noalloc. */
#define TQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Device.  tq_decode_attention for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, result and errors, without the
 * workspace arguments.  The workspace lives in a static device array of
 * TQ_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * until the process ends; the call allocates nothing (no hipMalloc / hipFree,
 * no allocating library routine).  Sizes whose workspace
 * (tq_decode_workspace_bytes) exceeds that return TQ_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array (the
 * query preparation of each call rewrites what the call reads), so calls that
 * overlap on one GPU (on different streams, or from different threads) race;
 * serialise them.  The first call on a device looks up the array's address
 * on that device (hipGetSymbolAddress); a failure there is TQ_ERR_HIP. */
tq_status tq_decode_attention_noalloc(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                      const float* q, int32_t batch, int32_t n_q_heads,
                                      const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                                      float scale, float* out, void* stream);

/* Human-readable name of a status code (static storage). */
const char* tq_status_string(tq_status status);

/* Thread-local detail message of the last failing call on this thread ("" if
 * none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
