/*
 * aatc.h - C ABI of the MI355X transform-coded KV cache (Attention-Aware Transform
 * Coding, AATC).
 *
 * The method (pages: "KV Cache Compression Through the Lens of Transform Coding",
 * abstract and Methodology; "Attention-Aware Transform Coding Guide", sections
 * "Decorrelation via the Karhunen-Loeve Transform", "Optimal Bit Allocation via
 * Reverse Water-Filling" and "Theorem: Additive Error Decomposition"; "Spend Bits
 * Where Queries Look" abstract for the fixed per-token bit count):
 *   calibrate: per (layer, kv-head) statistics -> KLT bases U_K, U_V, attention-aware
 *              channel weights, integer bits per channel by reverse water-filling under
 *              an average bits/element budget, scalar quantizer steps;
 *   encode:    bf16 K, V -> KLT coefficients -> per-channel codes -> packed tiles with a
 *              fixed number of bits per token;
 *   decode_attention: queries scored in the key transform domain (q' = U_K^T q) straight
 *              from the packed cache, online softmax, value coefficients accumulated and
 *              inverse-transformed once per query head.
 *
 * Conventions
 *   - Every function returns an int status: AATC_OK (0) or a negative AATC_ERR_* code;
 *     aatc_last_error() gives a thread-local message for the last failure.
 *   - Argument errors are detected before anything is enqueued; on error nothing is
 *     launched.  Device faults surface at the caller's next synchronisation.
 *   - The caller owns all device memory and streams ("stream" is a hipStream_t passed
 *     as void*; NULL is the null stream).  The library allocates host memory only (the
 *     codebook) and never synchronises a stream.  Device pointers must be 16-byte
 *     aligned.  A codebook is immutable once created and may be shared across threads.
 *   - head_dim d is 64 or 128; the query group size G = H_q / H_kv is 1..16; the budget
 *     B = 2 * d * avg_bits bits per token and kv-head must be a multiple of 8.
 *   - Matrices are row-major.  A basis U is d x d with U[i*d + j] = component i of basis
 *     vector j (coefficients are c = (x - mu) U).
 */
#ifndef AATC_H
#define AATC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AATC_VERSION 1
#define AATC_LAYOUT_VERSION 2

#define AATC_OK 0
#define AATC_ERR_INVALID_ARG (-1)
#define AATC_ERR_UNSUPPORTED (-2)
#define AATC_ERR_BUDGET (-3)
#define AATC_ERR_STATS (-4)
#define AATC_ERR_NO_CONVERGENCE (-5)
#define AATC_ERR_CAPACITY (-6)
#define AATC_ERR_WORKSPACE (-7)
#define AATC_ERR_HIP (-8)
#define AATC_ERR_IO (-9)
#define AATC_ERR_VERSION (-10)

/* Opaque host-side codebook: bases, bits and steps of n_layers * n_kv heads. */
typedef struct aatc_codebook aatc_codebook;

/* Calibration statistics of one (layer, kv-head); caller-owned arrays.
 * mu_k, mu_v: [d] channel means; sigma_k, sigma_v: [d*d] centred covariances (1/N);
 * m_q: [d*d] attention-weighted query moment mean_q g(q) q q^T with
 *      g(q) = sum_i A_i^2 ||v_i - o(q)||^2 over the calibration tokens;
 * gamma_v: mean_q sum_i A_i^2.  (Pages: the KLT section's channel covariances; the
 * theorem's key and value weights, read as expectations over calibration queries.) */
typedef struct {
    const double* mu_k;
    const double* mu_v;
    const double* sigma_k;
    const double* sigma_v;
    const double* m_q;
    double gamma_v;
} aatc_head_stats;

/* Calibration parameters.  avg_bits: average bits per cached element (the budget of the
 * reverse water-filling section, sum_j R_j = d * avg_bits per tensor); max_bits: per
 * channel cap (1..8); joint: 1 = keys and values share one budget of 2*d*avg_bits bits
 * per token (one water level for the sum D_K + D_V of the theorem), 0 = d*avg_bits each;
 * max_sweeps: Jacobi sweep limit of the eigensolver (0 = default 60);
 * key_transform: 0 = KLT of the key covariance (orthogonal U_K), 1 = attention-optimal
 * non-orthogonal transform T_K = M_Q^{1/2} R, R the eigenvectors of
 * M_Q^{1/2} Sigma_K M_Q^{1/2}, under which the attention-aware key distortion is the MSE of
 * the coefficients ("Spend Bits Where Queries Look", abstract; M_Q gets a ridge of 1e-6 of
 * its mean eigenvalue).  Values always use the KLT.
 * key_quantizer: 0 = scalar (per-channel widths from the water-filling), 1 = vector
 * quantization ("Spend Bits Where Queries Look", abstract): the d*avg_bits key bits of a
 * token become d*avg_bits/8 one-byte indices, one per group of 4 coefficients, into a
 * 256-word codebook per group.  Needs joint = 0, avg_bits <= 2 and d*avg_bits a multiple
 * of 32.  The 4 n_g coefficients of largest weight x_j are coded (the rest reconstruct to
 * the mean), grouped greedily toward equal volume prod x_j (largest weight first, into the
 * unfilled group of smallest sum of log(x_j / x_min)); each codebook is vq_iters (0 = 20)
 * rounds of Lloyd's algorithm (initial words: the first 256 points) on the points
 * vq_normals[n] * sqrt(x_j), n < vq_n_train, in the weighted domain u_j = sqrt(w_j) c_j
 * (w_j = x_j / lambda_j), where the attention-aware key distortion is plain MSE.
 * vq_normals: vq_n_train >= 256 rows of 4 standard normal draws (host, caller-owned),
 * ignored for scalar keys. */
typedef struct {
    double avg_bits;
    int32_t max_bits;
    int32_t joint;
    int32_t max_sweeps;
    int32_t key_transform;
    int32_t key_quantizer;
    int32_t vq_iters;
    const double* vq_normals;
    int64_t vq_n_train;
} aatc_calib_params;

/* Device-side cache descriptor.  data: caller-allocated device memory of
 * aatc_cache_bytes() bytes, zero-filled before first use.  The cache of
 * (layer, seq, kv-head) is a run of ceil(max_tokens/64) tiles of 64 token slots;
 * tile t lives at byte (((layer*n_seqs + seq)*n_kv + head)*n_tiles + t) * tile_bytes.
 * Inside a tile (layout version 2): a token's key record (B_K bits, a multiple of 32)
 * and value record (B_V bits, a multiple of 8) hold the channel codes as byte-aligned
 * fields (placement: widest channel first into the first byte with room; channels that
 * fit nowhere are cut to fill the remaining bits; bytes renumbered by decreasing field
 * count).  The key block (8*B_K bytes) is word-major: record word r of slot s is block
 * word 64r + s.  The value block (next 8*B_V bytes) is byte-major: record byte q of
 * slot s is block byte 64q + s.  Written bytes carry bit 7 inverted; unwritten slots
 * are zero. */
typedef struct {
    void* data;
    int32_t n_layers;
    int32_t n_seqs;
    int64_t max_tokens;
} aatc_cache;

/* ---- version and errors ------------------------------------------------------------ */
int aatc_version(void);                     /* AATC_VERSION */
int aatc_layout_version(void);              /* AATC_LAYOUT_VERSION */
const char* aatc_status_string(int status); /* static string for a status code */
const char* aatc_last_error(void);          /* thread-local detail of the last failure */

/* ---- host calibration ---------------------------------------------------------------- */

/* Statistics of one (layer, kv-head) from host samples (float32, row-major):
 * K, V [n x d] calibration keys/values, Q [nq x d] calibration queries of the G query
 * heads of the group, pooled.  Attention of every query over the n tokens is exact and
 * non-causal.  Outputs are caller-allocated: mu_k, mu_v [d]; sigma_k, sigma_v, m_q [d*d];
 * gamma_v [1].  Errors: INVALID_ARG (null pointer, n < 2, nq < 1, bad d), STATS
 * (non-finite input).  Runs on host threads. */
int aatc_stats_from_samples(int32_t d, const float* K, const float* V, int64_t n,
                            const float* Q, int64_t nq, double* mu_k, double* mu_v,
                            double* sigma_k, double* sigma_v, double* m_q, double* gamma_v);

/* Calibration ("Attention-Aware Transform Coding Guide": "Decorrelation via the
 * Karhunen-Loeve Transform" for the bases, "Optimal Bit Allocation via Reverse
 * Water-Filling" for the weights, the water level and the integer bits; "KV Cache
 * Compression Through the Lens of Transform Coding", Methodology, for the
 * attention-aware key and value weights; "Spend Bits Where Queries Look", abstract, for
 * the fixed bit count per token that the exact integer total keeps).
 * Calibrate n_layers * n_kv heads (stats indexed layer*n_kv + head): eigendecomposition of
 * both covariances (eigenvalues descending; each eigenvector's largest-magnitude entry
 * positive), channel weights x_K = lambda_K (U_K^T M_Q U_K)_jj / d and
 * x_V = lambda_V gamma_V, integer bits in [0, max_bits] with an exact total per token
 * (greedy on marginal gains x_j 4^-k; ties: keys, then lower channel, then lower k), and
 * steps step_b * sqrt(lambda_j) of the Gaussian-MSE-optimal 2^b-level uniform quantizer.
 * *out is allocated by the library (free with aatc_codebook_free).
 * Errors: INVALID_ARG, BUDGET (2*d*avg_bits not a multiple of 8, or out of range),
 * STATS (non-finite or non-PSD input), NO_CONVERGENCE (eigensolver). */
int aatc_calibrate(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                   const aatc_head_stats* stats, const aatc_calib_params* params,
                   aatc_codebook** out);

/* Build a codebook from explicit per-head arrays (e.g. produced by another calibration
 * tool): U_k, U_v [n_heads][d][d] float64 - coefficients are c = (x - mu) U, so U_v must be
 * orthogonal (the value reconstruction uses U_v^T) while U_k may be any invertible key
 * transform (queries are transformed by U_k^{-1}, computed here in fp64; INVALID_ARG when
 * singular); mu_k, mu_v [n_heads][d] float64; bits_k,
 * bits_v [n_heads][d] int32 in [0,8]; step_k, step_v [n_heads][d] float32 (> 0 where
 * bits > 0).  Every head must have the same total bits per token (a multiple of 8), with
 * key bits a multiple of 32.
 * Errors: INVALID_ARG, BUDGET. */
int aatc_codebook_create(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                         const double* U_k, const double* U_v, const double* mu_k,
                         const double* mu_v, const int32_t* bits_k, const int32_t* bits_v,
                         const float* step_k, const float* step_v, aatc_codebook** out);

/* Build a codebook with vector-quantized keys from explicit arrays.  Arguments as for
 * aatc_codebook_create, except for the keys: n_groups (a multiple of 4, 4*n_groups <= d)
 * groups; vq_chan [n_heads][n_groups][4] int32 key channels (distinct within a head);
 * vq_scale [n_heads][d] float32 s_j > 0 for coded channels; vq_cent
 * [n_heads][n_groups][256][4] float32 codewords in the weighted domain u = s c.
 * Encoding: index = argmin over words z of (t0 t0 + t1 t1) + (t2 t2 + t3 t3), t_k =
 * fp32(c_k s_k) - z_k, every operation rounded to fp32, lowest index on ties; decoding
 * c_j = z_k / s_j.  A token's key record is n_groups bytes (byte g = index of group g).
 * Errors: INVALID_ARG, BUDGET. */
int aatc_codebook_create_vq(int32_t d, int32_t n_layers, int32_t n_kv, int32_t group,
                            const double* U_k, const double* U_v, const double* mu_k,
                            const double* mu_v, int32_t n_groups, const int32_t* vq_chan,
                            const float* vq_scale, const float* vq_cent, const int32_t* bits_v,
                            const float* step_v, aatc_codebook** out);

/* Vector-quantized keys of one head: *n_groups (0 for scalar keys) and, where the
 * pointers are non-NULL and the head has them, vq_chan [n_groups*4], vq_scale [d],
 * vq_cent [n_groups*256*4] in the layout of aatc_codebook_create_vq. */
int aatc_codebook_vq(const aatc_codebook* cb, int32_t head, int32_t* n_groups, int32_t* vq_chan,
                     float* vq_scale, float* vq_cent);

/* Geometry of a codebook; any output pointer may be NULL.  total_bits = bits per token
 * and kv-head (keys and values); tile_bytes = 8 * total_bits. */
int aatc_codebook_info(const aatc_codebook* cb, int32_t* d, int32_t* n_layers,
                       int32_t* n_kv, int32_t* group, int32_t* total_bits,
                       int32_t* tile_bytes);

/* Copy out one head's calibration results (any pointer may be NULL): U_k, U_v [d*d],
 * lam_k, lam_v, mu_k, mu_v, x_k, x_v [d] float64; bits_k, bits_v [d] int32;
 * step_k, step_v [d] float32; theta [1] (continuous water level, 0 if not calibrated). */
int aatc_codebook_head(const aatc_codebook* cb, int32_t head, double* U_k, double* U_v,
                       double* lam_k, double* lam_v, double* mu_k, double* mu_v,
                       double* x_k, double* x_v, int32_t* bits_k, int32_t* bits_v,
                       float* step_k, float* step_v, double* theta);

/* Layout of one head's records: the byte-aligned fields of the key (which = 0) or value
 * (which = 1) record sorted by (byte, bit position), each packed as
 * chan | width << 8 | shift << 12 | pos << 16 | byte << 20 (the field holds code bits
 * [shift, shift + width) of channel chan at bits [pos, pos + width) of record byte
 * `byte`).  *n = number of fields; out may be NULL, else it holds at least 384 entries.
 * Errors: INVALID_ARG. */
int aatc_codebook_fields(const aatc_codebook* cb, int32_t head, int32_t which, uint32_t* out,
                         int32_t* n);

/* Persist / restore a codebook (versioned binary file with checksum).
 * Errors: IO, VERSION (layout or format mismatch, checksum failure). */
int aatc_codebook_save(const aatc_codebook* cb, const char* path);
int aatc_codebook_load(const char* path, aatc_codebook** out);
void aatc_codebook_free(aatc_codebook* cb);

/* ---- device side ------------------------------------------------------------------- */

/* Bytes of the device blob (bases, steps, bias vectors and kernel tables of all heads). */
int aatc_codebook_device_bytes(const aatc_codebook* cb, size_t* bytes);

/* Copy the blob to caller-allocated device memory d_blob (bytes >= device_bytes) with an
 * asynchronous copy on `stream`; the codebook must stay alive until the copy completes.
 * Errors: INVALID_ARG, WORKSPACE (too small), HIP. */
int aatc_codebook_upload(const aatc_codebook* cb, void* d_blob, size_t bytes, void* stream);

/* Bytes of a cache for n_layers x n_seqs sequences of up to max_tokens tokens. */
int aatc_cache_bytes(const aatc_codebook* cb, int32_t n_layers, int32_t n_seqs,
                     int64_t max_tokens, size_t* bytes);

/* Encoder ("Attention-Aware Transform Coding Guide", "Decorrelation via the
 * Karhunen-Loeve Transform": coefficients c = (x - mu) U; its code listing, read as a
 * per-channel uniform scalar quantizer at the allotted width; "Spend Bits Where Queries
 * Look", abstract: a fixed number of bits per token, which the 64-token tiles of
 * 8 * B bytes keep).
 * Append n_tokens tokens to each of n_seqs sequences of one layer.
 * seq_ids [n_seqs], start_pos [n_seqs]: host arrays; sequence s writes token slots
 * start_pos[s] .. start_pos[s]+n_tokens-1.  K, V: device bf16 [n_seqs][n_tokens][n_kv][d]
 * (contiguous).  The slots being written are rebuilt; the other slots of a partially
 * filled tile are kept (the tile is read, merged and written back).
 * Arithmetic: u = x (W_hi + W_lo) + (2^(b-1) - 1/2 - mu (W_hi + W_lo)) with W = U scaled
 * per channel by the fp32 reciprocal step and W_hi/W_lo its bf16 split (bf16 MFMA, fp32
 * accumulation, the start value rounded once from fp64; above 6.5 bits/element a third
 * bf16 term W_mid = W - W_hi - W_lo joins, for codebooks whose narrow cells the two-term
 * rounding would flip more than 1e-4 of the codes of); code = u clamped to
 * [0, 2^b - 1] and rounded to nearest, ties to even.  That is the quantizer of
 * aatc_encode_coeffs, floor(c/step) + 2^(b-1), wherever c/step is not within the fp32
 * rounding of this arithmetic of a cell edge.
 * Errors: INVALID_ARG, CAPACITY (start_pos + n_tokens > max_tokens), HIP. */
int aatc_encode(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                const int64_t* start_pos, int64_t n_tokens, const uint16_t* K,
                const uint16_t* V, void* stream);

/* Quantize and pack given KLT coefficients ("Attention-Aware Transform Coding Guide",
 * code listing, read as a midrise uniform quantizer per channel; the 2^b-level step that
 * minimizes the mean squared error of a unit Gaussian, scaled by sqrt(lambda_j), is this
 * library's reading of the same section's quantizer).  Skips the projection: coeffs device float32
 * [n_tokens][n_kv][2][d] (keys then values, KLT channel order) for one (layer, seq)
 * starting at slot start_pos.  Code of channel j with b > 0 bits:
 * t = fp32(c * fp32(1/step_j)) (one rounding), code = clamp(floor(t) + 2^(b-1), 0, 2^b-1).
 * Non-finite coefficients give unspecified codes.  Errors as aatc_encode. */
int aatc_encode_coeffs(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                       int32_t layer, int32_t seq, int64_t start_pos, int64_t n_tokens,
                       const float* coeffs, void* stream);

/* Workspace bytes for aatc_decode_attention with n_seqs sequences of length <= max_len: a
 * 1 KiB block of arrival counters followed by the split partials. */
int aatc_decode_workspace_bytes(const aatc_codebook* cb, int32_t n_seqs, int64_t max_len,
                                size_t* bytes);

/* One decode step of one layer: out[s][h] = softmax(q_h K_hat^T / sqrt(d)) V_hat over the
 * first seq_lens[s] cached tokens of sequence seq_ids[s] (no mask), query head h reading
 * kv-head floor(h / G).  seq_ids [n_seqs] int32 and seq_lens [n_seqs] int64 are DEVICE
 * arrays (1 <= seq_lens[s] <= max_len <= max_tokens); max_len (host) sizes the grid.
 * q: device bf16 [n_seqs][H_q][d]; out: device float32 [n_seqs][H_q][d]; workspace:
 * device scratch of aatc_decode_workspace_bytes() bytes (256-byte aligned) for the split
 * partials and their arrival counters.  It must be zero-filled once before its first use
 * (e.g. at allocation); every call leaves the counters at zero again.  Calls that share a
 * workspace must not overlap in time (same stream, or ordered).  The split decode over the
 * packed tiles runs as one kernel on `stream` (each workgroup transforms the queries
 * itself; the last workgroup of each (sequence, kv-head) to finish merges the partials and
 * applies the inverse transform), or, when a call has more than 256 (sequence, kv-head)
 * pairs, more than 64 workgroups per pair or more than 32 KiB of partials per pair (a large
 * merge is faster spread over many CUs), as that kernel followed by a merge kernel
 * ("KV Cache Compression Through the Lens of Transform Coding", Methodology;
 * "Attention-Aware Transform Coding Guide", KLT section: q.k = (U_K^T q).(U_K^T k)).
 * At most 65535 sequences per call (CAPACITY beyond).
 * With vector-quantized keys (aatc_codebook_create_vq, key_quantizer = 1) the scores come
 * from per-(query head, group) tables over the codebooks (a token's score is the sum of
 * its groups' entries); the workspace is the same and the merge kernel always follows.
 * Errors: INVALID_ARG, CAPACITY, WORKSPACE, HIP; UNSUPPORTED (before anything is enqueued,
 * also from aatc_decode_workspace_bytes) when a head's tiles and operand scratch need more
 * LDS than a CU holds: at d = 128 above 7.5 bits/element. */
int aatc_decode_attention(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                          int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                          const int64_t* seq_lens, int64_t max_len, const uint16_t* q,
                          float* out, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for aatc_decode_attention_layers over layers [layer0, layer0 + n_layers)
 * with n_seqs sequences of length <= max_len (the largest any of its launches needs).
 * Errors: INVALID_ARG, UNSUPPORTED (vector-quantized keys; a variant as for
 * aatc_decode_attention_layers). */
int aatc_decode_layers_workspace_bytes(const aatc_codebook* cb, int32_t layer0, int32_t n_layers,
                                       int32_t n_seqs, int64_t max_len, size_t* bytes);

/* aatc_decode_attention for the same sequences in n_layers consecutive layers
 * [layer0, layer0 + n_layers) at once, for callers that hold every layer's queries (the
 * attention of each layer is the one defined for aatc_decode_attention: "Attention-Aware
 * Transform Coding Guide", Formal Attention Distortion Model and KLT section).  q and out
 * are [n_layers][n_seqs][H_q][d] (layer-major); seq_ids / seq_lens as for one layer and
 * shared by all layers.  The layers run as few launches: one per run of consecutive layers
 * whose heads take the same decode variant, each run's (layer, sequence, kv-head) triples
 * splitting the CUs between them, so the fixed cost of a launch is paid once per run
 * rather than once per layer.  Results are those of one aatc_decode_attention call per
 * layer.  In a model the layers of one step follow each other (a layer's queries depend on
 * the previous layer's output); per-layer calls are the path for that.  Workspace:
 * aatc_decode_layers_workspace_bytes() bytes, rules as for aatc_decode_attention (the runs
 * use it one after another on `stream`).  At most 65535 (layer, sequence) slots.
 * Errors: INVALID_ARG (also layers outside the codebook), CAPACITY, WORKSPACE, HIP;
 * UNSUPPORTED with vector-quantized keys.  Every argument and run is checked before the
 * first launch. */
int aatc_decode_attention_layers(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                 int32_t layer0, int32_t n_layers, int32_t n_seqs,
                                 const int32_t* seq_ids, const int64_t* seq_lens, int64_t max_len,
                                 const uint16_t* q, float* out, void* workspace, size_t ws_bytes,
                                 void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops that forbid allocation): aatc_decode_attention with its partials and arrival
 * counters in an 8 MiB device array of the library's own (one per GPU, held until the
 * process ends) instead of a caller workspace; nothing is allocated.  The counters are zero
 * when the library is loaded and every call leaves them at zero.  All calls on one GPU
 * share the array: calls that overlap in time on the same GPU race (issue them on one
 * stream, or order them).  Other arguments as aatc_decode_attention.
 * Errors: CAPACITY when the call needs more than 8 MiB of partials
 * (aatc_decode_workspace_bytes > 8 MiB), otherwise as aatc_decode_attention. */
int aatc_decode_attention_static(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                 int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                 const int64_t* seq_lens, int64_t max_len, const uint16_t* q, float* out,
                                 void* stream);

/* One generation step of one layer: append one token per sequence, then decode over the
 * grown cache, in the same launch.  k_new, v_new: device bf16 [n_seqs][n_kv][d] (16-byte
 * aligned); the token of sequence s is written at slot seq_lens[s] (device array: the
 * tokens cached before the call) with the codes aatc_encode would write for it, and the
 * attention runs over seq_lens[s] + 1 tokens (each limited to max_len and max_tokens; a
 * slot past that limit is neither written nor attended).  The caller advances seq_lens
 * afterwards.  Other arguments, workspace and errors as aatc_decode_attention.  The
 * workgroup that owns the token's tile codes it (the encoder's MFMA projection and
 * quantizer) and places its records in its copy of the tile, so the step needs no ordering
 * between the write and the tile's stream ("Spend Bits Where Queries Look", abstract:
 * decoding reads the whole cache at every step).  UNSUPPORTED for codebooks with
 * vector-quantized keys (append with aatc_encode, then decode). */
int aatc_decode_attention_append(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                 int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                 const int64_t* seq_lens, int64_t max_len, const uint16_t* k_new,
                                 const uint16_t* v_new, const uint16_t* q, float* out, void* workspace,
                                 size_t ws_bytes, void* stream);

/* ---- measurement helpers ----------------------------------------------------------- */

/* Overwrite `bytes` of caller-allocated device memory with a streaming write (used to
 * evict the device's last-level cache between timed repetitions).  Errors: HIP. */
int aatc_flush_write(void* d_buf, size_t bytes, void* stream);

/* Streaming-read probe: one launch on `stream` reads `bytes` of caller-allocated device
 * memory d_src the way a decode step reads its cache, to measure the HBM read rate the
 * decode kernel can be held to ("Spend Bits Where Queries Look", abstract: decoding is
 * bandwidth-bound).  mode 0: plain 16-byte register loads over the whole buffer; mode 1:
 * tiles of tile_bytes bytes (a multiple of 256, at most 6656) streamed into LDS like the
 * decode kernel's ring (one 768-thread workgroup per CU, even share, two slots per wave),
 * over the first floor(bytes / tile_bytes) tiles (at most 2^31 - 1 bytes).  d_sink: 16
 * bytes of device memory the probe may write (it never does for real data: the loaded
 * words only feed a checksum).  Both pointers 16-byte aligned.
 * Errors: INVALID_ARG, CAPACITY, HIP. */
int aatc_read_probe(const void* d_src, size_t bytes, int32_t mode, int32_t tile_bytes, void* d_sink,
                    void* stream);

/* Kernel timing for measurement: after aatc_profile_begin(n) the next n calls of
 * aatc_decode_attention (any thread, current device) record a pair of device events
 * around their split-decode kernel on the call's stream (the query-preparation kernel
 * before it is not included).  aatc_profile_end waits for those events and writes the
 * kernel durations in milliseconds to ms[0 .. *n_out) (ms holds the n given to begin),
 * then releases the events.  Meant for benchmarks, not for concurrent production use.
 * Errors: INVALID_ARG (n < 1, profiling already active / not active), HIP. */
int aatc_profile_begin(int32_t n);
int aatc_profile_end(float* ms, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* AATC_H */
