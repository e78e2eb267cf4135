/*
 * kvtc.h - C ABI of libkvtc, KV-cache transform coding on AMD Instinct MI355X
 * (gfx950).
 *
 * The method is the one on the page "KV Cache Transform Coding for Compact
 * Storage in LLM Inference" (gist.science, paper 2511.01815), section 2:
 *   2A calibration   : PCA basis by SVD, shared across heads and computed once;
 *                      s sink tokens and w window tokens stay uncompressed;
 *                      dynamic-programming bit widths under a bit budget;
 *                      a group of components shares a scale and a shift.
 *   2B compression   : subtract the mean, multiply by V, quantize, pack
 *                      (the DEFLATE stage is on the host and only reports the
 *                      lossless ratio, see kvtc_deflate).
 *   2C decompression : dequantize, multiply by V^T, add the mean, layer by
 *                      layer.
 * The page fixes no formats or arithmetic; the byte formats and rounding rules
 * implemented here are:
 *   widths       one width b in 0..max_bits (<= 8) per group of G consecutive
 *                components (G = group, 16 or 32 in practice, a multiple of 8);
 *                cost per compressed token: G*b bits + 64 bits (fp32 shift and
 *                fp32 scale) for every group with b > 0; budget
 *                floor(bits_per_value * F) bits; ties go to fewer bits, then to
 *                the lexicographically larger widths.
 *   quantizer    per (token, active group): shift = min c, scale = max c - min c
 *                (fp32), q = clamp(rint_even(fp32(c - shift) * fp32(k/scale)),
 *                0, k) with k = 2^b - 1 and q = 0 when scale == 0.
 *   projection   c_j = sum_f (x_f - mu32_f) V'_fj with V' = bf16_rne(V32),
 *                the centred token taken exactly. On the device: d = x - mu_hi
 *                in fp32 with mu_hi = bf16_rne(mu32) (exact for bf16 tokens
 *                within a factor 2^8 of the mean), split into bf16 terms
 *                (two for bf16 input, three for f32) that are each multiplied
 *                on bf16 MFMA with fp32 accumulation started at
 *                -(mu32 - mu_hi) V'; the rounding error scales with |x - mu|,
 *                so a code may differ by one step from the exact sum near a
 *                rounding boundary whatever the size of the mean. A bf16 slot
 *                whose mean is no larger than its spread (|mu32|^2 <= sum of
 *                the calibration's covariance eigenvalues) folds the mean
 *                instead: the stored token is one exact bf16 operand and the
 *                accumulation starts at -mu32 V' (fp64, rounded once); its
 *                rounding error scales with |x|, within a factor of about
 *                sqrt(2) of |x - mu| there (kvtc_slot_info.folded_mean). A
 *                slot finished (calibrated or loaded) while the environment
 *                variable KVTC_ENCODE_CENTRED is "1" stays centred.
 *   dequantize   c_hat = shift + q * fp32(scale / k); dropped groups give 0;
 *                x_hat = mu32 + sum_j c_hat_j V'_j.
 *   stream       64-byte header ("KVTC", u16 version=1, u8 dtype, u8 kind,
 *                u32 layer, T, F, s', w', T_c, u16 G, u16 n_act,
 *                u32 record_bytes, u64 slot_id, zeros), then the raw rows
 *                [0, s') and [T - w', T), then T_c records of record_bytes;
 *                s' = min(s, T), w' = min(w, T - s'), T_c = T - s' - w'.
 *   record       n_act x (f32 shift, f32 scale), then per active group its G
 *                codes, code j in bits [j*b, j*b + b) of the group's G*b/8-byte
 *                chunk, least significant bit first.
 *   artifact     see kvtc_save.
 * All multi-byte fields are little-endian.
 *
 * Memory and ownership: the caller owns every device buffer (KV tensors,
 * streams, device state, workspace, staging, block tables) and every stream.
 * The library owns only the host-side codec. It never allocates device memory;
 * it enqueues work only on the stream it is given and never synchronises it,
 * except kvtc_upload and kvtc_read_device_status, which say so.
 *
 * Errors: every call returns kvtc_status. Argument, shape, capacity and
 * calibration errors are found on the host; the call then enqueues nothing
 * and kvtc_last_error() describes the problem. Stream-content errors (magic,
 * version, slot id, shape fields) are found on the device: the failing job's
 * status word in the workspace is set and none of its output rows are written.
 *
 * Threads: a codec may be used from several host threads and streams at once
 * for encode and decode if each concurrent call has its own workspace.
 * kvtc_calibrate may run concurrently on distinct (layer, kind) slots.
 */
#ifndef KVTC_H
#define KVTC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVTC_OK = 0,
  KVTC_E_INVALID = -1,         /* bad argument, shape or parameter            */
  KVTC_E_CAPACITY = -2,        /* an output or workspace buffer is too small  */
  KVTC_E_CORRUPT = -3,         /* malformed artifact or stream                */
  KVTC_E_MISMATCH = -4,        /* stream does not belong to this job/codec    */
  KVTC_E_NOT_CALIBRATED = -5,  /* (layer, kind) has no calibration            */
  KVTC_E_HIP = -6,             /* a HIP runtime call failed                   */
  KVTC_E_UNSUPPORTED = -7      /* valid but outside the library's limits      */
} kvtc_status;

typedef enum { KVTC_F32 = 0, KVTC_BF16 = 1 } kvtc_dtype;
typedef enum { KVTC_K = 0, KVTC_V = 1 } kvtc_kind;

/* Codec parameters. F = kv_heads * head_dim; feature h*head_dim + i is element
 * i of head h (heads concatenated, the basis is shared across heads). */
typedef struct {
  int32_t n_layers;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t sink;            /* s: oldest tokens kept verbatim                 */
  int32_t window;          /* w: newest tokens kept verbatim                 */
  int32_t group;           /* G: components per microscale group             */
  int32_t max_bits;        /* largest width, 0..8                            */
  float bits_per_value;    /* budget per compressed value, e.g. 16/ratio     */
  int32_t dtype;           /* kvtc_dtype of the KV tensors                   */
} kvtc_params;

typedef struct kvtc_codec kvtc_codec;

/* One tensor of work: the K or V cache of one layer, [n_tokens, F] rows.
 *   encode:  src = KV rows (device, params.dtype), dst = stream (device).
 *   decode:  src = stream (device), dst = KV rows (device, out dtype).
 * src_capacity bounds what the kernels read at src: n_tokens rows for encode
 * (and for kvtc_pack's passthrough rows), kvtc_encoded_bytes(n_tokens) for
 * decode and kvtc_unpack; a smaller value is rejected with KVTC_E_CAPACITY
 * before anything is launched.
 * block_table (device, int32, decode only): when non-NULL, token t is written
 * to physical row block_table[t / block_size] * block_size + t % block_size
 * of dst (a paged cache of [n_blocks, block_size, F]); dst_capacity bounds the
 * physical rows. */
typedef struct {
  int32_t layer;
  int32_t kind;
  int64_t n_tokens;
  const void* src;
  size_t src_capacity;     /* bytes readable at src                          */
  void* dst;
  size_t dst_capacity;     /* bytes available at dst                         */
  const int32_t* block_table;
  int32_t block_size;
  int32_t n_blocks;        /* physical blocks in dst when paged              */
} kvtc_job;

/* Per-slot calibration summary. */
typedef struct {
  int32_t calibrated;
  int32_t n_act;           /* groups with b > 0                              */
  int32_t r_eff;           /* n_act * G active components                    */
  int32_t record_bytes;    /* bytes per compressed token                     */
  uint64_t slot_id;        /* FNV-1a 64 of the slot's serialized bytes       */
  uint8_t widths[512];     /* width per group (F/G entries); with a width
                              per component, each group's largest            */
  int32_t per_component;   /* 1: a width per component (see kvtc_calibrate_set) */
  int32_t folded_mean;     /* 1: the encode multiplies the token as stored and
                              subtracts mu32 V' (bf16 codecs whose |mu32|^2 is
                              at most the sum of the covariance eigenvalues);
                              0: it centres each token first (see projection) */
} kvtc_slot_info;

/* Largest active component count the kernels accept. */
#define KVTC_MAX_REFF 256
/* Largest number of jobs per call. */
#define KVTC_MAX_JOBS 4096

const char* kvtc_version(void);
/* Last error message of the calling thread ("" if none). */
const char* kvtc_last_error(void);

/* Create a codec (host memory only). Fails with KVTC_E_INVALID unless
 * F % G == 0, G % 8 == 0, 0 <= max_bits <= 8, bits_per_value >= 0,
 * F / G <= 512 and dtype is KVTC_F32 or KVTC_BF16. */
kvtc_status kvtc_create(const kvtc_params* params, kvtc_codec** out);
void kvtc_destroy(kvtc_codec* codec);

/* Calibrate one (layer, kind) on the host (section 2A): rows [s, n - w) of
 * host_kv ([n_tokens, F], params.dtype storage, host memory, read only) give
 * the fp64 mean, the covariance, its eigenvectors (a Householder
 * tridiagonalisation and implicit QL iteration; the eigenvectors of the
 * covariance are the right singular vectors of the centred rows) sorted by
 * descending eigenvalue with the largest-magnitude entry of each made
 * positive, the empirical distortion D_g(b) of the quantizer on the
 * calibration coefficients, and the DP widths. n_tokens - s - w must be >= 1.
 * The widths keep at most KVTC_MAX_REFF / G active groups (the kernels'
 * limit): when the DP's optimum needs more, they minimise the distortion
 * under both the budget and that cap. Uses up to `threads` host threads
 * (0 = hardware concurrency). */
kvtc_status kvtc_calibrate(kvtc_codec* codec, int32_t layer, int32_t kind,
                           const void* host_kv, int64_t n_tokens, int32_t threads);

/* One tensor of a calibration set: [n_tokens, F] rows in params.dtype
 * storage, host memory, read only. */
typedef struct {
  int32_t layer;
  int32_t kind;
  const void* host_kv;
  int64_t n_tokens;
} kvtc_calib_input;

/* kvtc_calibrate_set flags. */
#define KVTC_CAL_SHARED_BASIS 1u  /* one basis per kind across the set's layers */
#define KVTC_CAL_GLOBAL_BUDGET 2u /* one bit budget across the whole set */
#define KVTC_CAL_COMPONENT_WIDTHS 4u /* a width per component inside each group */

/* Calibrate several (layer, kind) tensors in one call. The page on KV cache
 * transform coding finds one PCA basis reusable across layers and heads
 * (section 3, contributions) and places bits by a DP under a budget (section
 * 2A); the two flags apply these across tensors:
 *   KVTC_CAL_SHARED_BASIS: the tensors of one kind share one basis, the
 *     eigenvectors of the sum of their scatter matrices over the total row
 *     count, each tensor's rows [s, n - w) centred on its own mean first.
 *     Every tensor keeps its own mean, distortion table and widths; each
 *     slot stores its own copy of the basis, so streams, kernels and the
 *     artifact format are unchanged.
 *   KVTC_CAL_GLOBAL_BUDGET: the widths of all tensors are chosen together,
 *     minimising the sum of their distortion tables subject to the sum of
 *     their bits per token being at most n * floor(bits_per_value * F), with
 *     at most KVTC_MAX_REFF / G active groups per tensor. Ties: fewest total
 *     bits, then the most bits to the tensor earliest in (layer, kind) order,
 *     then kvtc_calibrate's rule inside each tensor.
 *   KVTC_CAL_COMPONENT_WIDTHS (not with the global budget): section 2A gives
 *     each principal component its own width; with this flag every
 *     component j of a group gets a width b_j in 0..max_bits while the group
 *     keeps one (shift, scale) per token, the min and range of all its G
 *     components. Component j is coded on k_j = 2^b_j - 1 levels,
 *     q = clamp(rint(fp32(c - shift) * fp32(k_j / scale)), 0, k_j), and
 *     decodes to shift + q * fp32(scale / k_j); b_j = 0 drops it (0). A
 *     group is active if any b_j > 0; its codes are packed in component
 *     order, code j at bit sum_{i<j} b_i of the group's chunk, which is
 *     ceil(sum_j b_j / 8) bytes; an active group costs 64 + 8 ceil(sum_j
 *     b_j / 8) bits. The widths minimise the sum of the components'
 *     empirical distortions within the budget (ties: fewest bits, then the
 *     largest width sum for the earliest group, then the largest widths
 *     first). Such slots serialize with mode 1 (see kvtc_save); every
 *     decode schedule, kvtc_decode_noalloc and the lossless stage take them
 *     (in launches of their own); the pack/unpack hooks return
 *     KVTC_E_UNSUPPORTED for them.
 * With no flag each tensor gets exactly kvtc_calibrate's result. A (layer,
 * kind) may appear at most once; the call is all or nothing (on error no slot
 * changes). Every tensor keeps to the kernels' cap of KVTC_MAX_REFF active
 * components as in kvtc_calibrate: with a width per component, when the
 * plain allocation has more than KVTC_MAX_REFF / G active groups, the widths
 * minimise the distortion under both the budget and that cap (same tie
 * order). Errors: KVTC_E_INVALID (bad arguments, unknown flags, too few
 * rows, duplicates). */
kvtc_status kvtc_calibrate_set(kvtc_codec* codec, const kvtc_calib_input* inputs, int32_t n,
                               uint32_t flags, int32_t threads);

kvtc_status kvtc_slot_info_get(const kvtc_codec* codec, int32_t layer, int32_t kind,
                               kvtc_slot_info* info);

/* Serialize every calibrated slot. With buf == NULL, only *written (the size
 * needed) is set. Format (little-endian): "KVTA", u32 version=1, i32 n_layers,
 * kv_heads, head_dim, sink, window, group, max_bits, f32 bits_per_value,
 * i32 dtype, i32 n_slots, then per slot in (layer, kind) order: "KVTS",
 * i32 layer, kind, F, G, n_act, r_eff, mode (0: a width per group, 1: a
 * width per component), u8 widths[F/G] (mode 0) or widths[F] (mode 1)
 * zero-padded to a multiple of 8, f32 mu32[F], f64 lambda[F], f32
 * V32[F][r_eff] (active groups' columns in component order), u64 slot_id =
 * FNV-1a 64 of the slot's preceding bytes. */
kvtc_status kvtc_save(const kvtc_codec* codec, void* buf, size_t cap, size_t* written);
/* Create a codec from artifact bytes (host memory); checks every slot id. */
kvtc_status kvtc_load(const void* buf, size_t n, kvtc_codec** out);

/* Device state: the operational basis in the layouts the kernels read, the
 * means and the per-slot descriptors. kvtc_upload copies it into the caller's
 * device buffer d_state (>= kvtc_device_state_bytes bytes, 256-byte aligned)
 * on `stream` and synchronises that stream before returning. Encode and decode
 * use the buffer of the last upload; re-upload after any new calibration. */
size_t kvtc_device_state_bytes(const kvtc_codec* codec);
kvtc_status kvtc_upload(kvtc_codec* codec, void* d_state, size_t bytes, hipStream_t stream);

/* Exact stream size for a tensor of n_tokens rows (0 if not calibrated). */
size_t kvtc_encoded_bytes(const kvtc_codec* codec, int32_t layer, int32_t kind,
                          int64_t n_tokens);
/* Workspace (device) for a call with up to max_jobs jobs: one 64-bit status
 * word per job (256-byte aligned), then a 256-byte sink that absorbs the
 * kernels' stores that have no destination row. Each launch stamps the words
 * it writes, so the workspace needs no clearing between calls;
 * kvtc_decode_restore reads the words kvtc_decode_unpack left. */
size_t kvtc_workspace_bytes(int32_t max_jobs);

/* Encode n_jobs tensors in one launch (section 2B). Each job's dst must hold
 * kvtc_encoded_bytes. d_ws: workspace for n_jobs jobs. The kernel is
 * persistent (at most two workgroups per CU, each over an equal range of
 * 32-token blocks); the environment variable KVTC_MAX_WORKGROUPS, if set to
 * a positive integer, caps that grid and the decode stage-2 grid (rounded
 * down to a multiple of 8, at least 8) and changes no result. */
kvtc_status kvtc_encode(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                        void* d_ws, hipStream_t stream);

/* Decode n_jobs streams (section 2C), writing out_dtype rows, in one of two
 * schedules that produce identical results, chosen by the workspace given:
 *  - ws_bytes >= kvtc_decode_workspace_bytes(jobs) (kvtc_workspace_bytes
 *    (n_jobs) followed by kvtc_staging_bytes(jobs)): the two-stage schedule
 *    below, stage 1 then stage 2 of each launch batch in turn, with the
 *    staging inside d_ws;
 *  - kvtc_workspace_bytes(n_jobs) <= ws_bytes < that: the fused schedule, one
 *    launch per batch (at most 32 jobs of one K-step count) that dequantizes
 *    each block of 32 records into MFMA operands in LDS and restores it, with
 *    no staging.
 * kvtc_decode_workspace_bytes is 0 if a job names an unknown or uncalibrated
 * (layer, kind); a smaller workspace gives KVTC_E_CAPACITY. Passthrough rows
 * are copied bit for bit when out_dtype equals the codec dtype (converted
 * with round-to-nearest-even otherwise). */
size_t kvtc_decode_workspace_bytes(const kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs);
kvtc_status kvtc_decode(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                        int32_t out_dtype, void* d_ws, size_t ws_bytes, hipStream_t stream);

/* kvtc_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc): the fused
 * schedule, with its status words and sink in a static device array of
 * kvtc_workspace_bytes(KVTC_MAX_JOBS) bytes (33 KiB; one copy per GPU, kept
 * until the process ends, its address looked up on the first call on each
 * device) instead of a caller's workspace. The call allocates nothing: it
 * clears this call's status words with a small kernel, decodes, and, if
 * d_status is not NULL, writes each job's kvtc_status to d_status[i] (device
 * memory, n_jobs int32) on `stream`. More than KVTC_MAX_JOBS jobs give
 * KVTC_E_CAPACITY. Every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other threads) race on it. */
kvtc_status kvtc_decode_noalloc(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                                int32_t out_dtype, int32_t* d_status, hipStream_t stream);

/* Two-stage decode for layer-by-layer pipelines (section 2C: decompression
 * can proceed layer by layer). Stage 1 validates headers, copies passthrough
 * rows to dst and turns every record into the operands of the
 * reconstruction: for each token the dequantized coefficients
 * c_hat = shift + q * fp32(scale / (2^b - 1)) divided by a power of two S_t
 * (chosen per token so the largest |c_hat| / S_t lies in [2^14, 2^15)) as
 * fp16, and S_t. Stage 2 forms S_t * (V' c) + mu for every compressed row and
 * writes it to dst. Both stages must see the same jobs, staging and
 * workspace. Staging layout per job (consecutive, each 256-byte aligned):
 * for each block of 32 compressed tokens, ks = ceil(r_eff / 16) x 64
 * fragments of 8 fp16 (fragment (s, l) holds components 16 s + 8 (l / 32)
 * .. + 8 of token l % 32 of the block; zero past r_eff and past the last
 * token), then 32 f32 S_t. kvtc_staging_bytes is 0 when no job has
 * compressed rows (d_staging may then be NULL) or when a job names an unknown
 * or uncalibrated (layer, kind). */
size_t kvtc_staging_bytes(const kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs);
kvtc_status kvtc_decode_unpack(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                               int32_t out_dtype, void* d_staging, size_t staging_bytes,
                               void* d_ws, hipStream_t stream);
kvtc_status kvtc_decode_restore(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                                int32_t out_dtype, const void* d_staging,
                                size_t staging_bytes, void* d_ws, hipStream_t stream);

/* Test hook: build the whole stream of one job from given codes
 * (u8 [T_c][r_eff], device) and shift/scale pairs (f32 [T_c][n_act][2],
 * device) with the encoder's own record packing; job.src supplies the
 * passthrough rows. */
kvtc_status kvtc_pack(kvtc_codec* codec, const kvtc_job* job, const void* d_codes,
                      const void* d_shift_scale, void* d_ws, hipStream_t stream);

/* Test hook: the inverse of kvtc_pack's record packing. Reads the records of
 * one job's stream (job.src; the header is not checked) into codes
 * (u8 [T_c][r_eff], device) and shift/scale pairs (f32 [T_c][n_act][2],
 * device); job.dst is not written. */
kvtc_status kvtc_unpack(kvtc_codec* codec, const kvtc_job* job, void* d_codes, void* d_shift_scale,
                        void* d_ws, hipStream_t stream);

/* Copy n_jobs status words from the workspace to host memory. This
 * synchronises `stream` first. Each word is KVTC_OK or a kvtc_status. */
kvtc_status kvtc_read_device_status(const void* d_ws, int32_t n_jobs, int32_t* status,
                                    hipStream_t stream);

/* Host DEFLATE (zlib, the given level) of n bytes of host memory, for the
 * lossless ratio of section 2B. With out == NULL only *out_len (an upper
 * bound) is set. */
kvtc_status kvtc_deflate(const void* in, size_t n, void* out, size_t cap, size_t* out_len,
                         int32_t level);

/* ------------------------------------------------------------------------
 * Lossless stage on the GPU. The KVTC page (section 2B) ends compression
 * with DEFLATE run on the GPU; this stage is a coder of our own in its
 * place that knows the stream layout. A KVTC stream is split into fields:
 *   P_j (j < esz, esz = 2 for bf16, 4 for f32): byte j of every passthrough
 *       element (rows [0, s') then [T - w', T)), alphabet 256;
 *   S_j, R_j (j < 4): byte j of every record's fp32 shifts, then scales,
 *       token-major then group, alphabet 256;
 *   Q_a (a < n_act): the codes of active group a, token-major then
 *       component, alphabet 2^b_a. With a width per component each code is
 *       read from its own b_j bits (a width-0 component gives 0) and b_a is
 *       the group's largest width; the decode packs each back into its own
 *       bits, the chunk's padding bits zero.
 * Each field has a static model: its histogram h over its alphabet, N = sum
 * h, n_p present symbols, M = 4096, f_s = 0 if h_s = 0 else
 * 1 + floor(h_s * (M - n_p) / N), the remainder M - sum f added to the most
 * frequent symbol (lowest index on ties), c_s = sum of f below s. Each field
 * is cut into chunks of 16384 symbols (the last one shorter), each coded by
 * rANS (J. Duda's asymmetric numeral systems; 32-bit states, L = 2^16,
 * 16-bit words) with 64 interleaved states: symbol i of a chunk belongs to
 * state i mod 64 and step i div 64. Encoding starts every state at L and
 * runs the steps from the last: each state with a symbol s emits its low 16
 * bits and shifts right by 16 if x >= f_s * 2^20, then
 * x = floor(x / f_s) * M + (x mod f_s) + c_s. A chunk's payload is the 64
 * final states (low word, high word), then the emitted words of step 0,
 * step 1, ..., inside a step by ascending state. Decoding runs the steps
 * from the first: slot = x mod M, s with c_s <= slot < c_s + f_s,
 * x = f_s * floor(x / M) + slot - c_s, then the states with x < L take the
 * next words in ascending order (x = x * 2^16 + w); every state ends at L.
 *
 * Container ("KVTZ", little-endian): u32 magic, u16 version = 1, u16
 * n_fields, u32 chunk symbols = 16384, u32 n_chunks, u64 stream bytes, u64
 * container bytes, u32 payload offset, zeros to byte 64; the stream's
 * 64-byte header; per field u32 n_symbols, u16 alphabet A, u16 0, u16 f[A];
 * u32 end[n_chunks] (each chunk's payload end relative to the payload
 * offset, chunks in field order); zeros to the payload offset (a multiple of
 * 16); the payloads; zeros to the container size (a multiple of 16).
 * ---------------------------------------------------------------------- */

/* Largest container of a (layer, kind) stream of n_tokens tokens (0 if
 * uncalibrated). */
size_t kvtc_lossless_bound(const kvtc_codec* codec, int32_t layer, int32_t kind, int64_t n_tokens);

/* Workspace bytes for kvtc_lossless_encode (encode != 0) or _decode of these
 * jobs (0 on a bad job): the status words, one u64 container size per job,
 * then per job its field symbols, models and (encode) per-chunk scratch:
 * about 3.4 times the stream for encode and 1.2 times for decode at 8192
 * tokens of 1024 bf16 features. */
size_t kvtc_lossless_workspace_bytes(const kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs,
                                     int32_t encode);

/* Stream -> container for each job: src is the KVTC stream (device,
 * src_capacity >= kvtc_encoded_bytes), dst the container (device,
 * dst_capacity >= kvtc_lossless_bound); both 16-byte aligned. The container
 * size of job i is stored in the workspace (kvtc_lossless_sizes) and in the
 * container's header. Host errors as for kvtc_encode (KVTC_E_CAPACITY for a
 * workspace below kvtc_lossless_workspace_bytes); the stream is not checked
 * (run kvtc_decode on it for that). Enqueued on `stream`, not synchronised. */
kvtc_status kvtc_lossless_encode(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs, void* d_ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Container -> stream for each job: src is the container (device,
 * src_capacity at least its container bytes, which the device checks, and
 * at least its tables, which the host checks), dst the stream (device,
 * dst_capacity >= kvtc_encoded_bytes). A container whose header, tables or
 * directory do not match the job's shape (KVTC_E_MISMATCH) or are
 * inconsistent, or whose payload does not decode exactly to its chunk
 * (KVTC_E_CORRUPT), sets the job's status word and no byte of its dst is
 * written. */
kvtc_status kvtc_lossless_decode(kvtc_codec* codec, const kvtc_job* jobs, int32_t n_jobs, void* d_ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Copy the n_jobs container sizes of the last kvtc_lossless_encode on this
 * workspace to host memory; synchronises `stream` first. */
kvtc_status kvtc_lossless_sizes(const void* d_ws, int32_t n_jobs, uint64_t* sizes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVTC_H */
