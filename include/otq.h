/*
 * otq.h - int4 KV-cache quantisation and decode attention computed directly
 * on the packed int4 cache, for AMD Instinct MI355X (gfx950).
 *
 * The method: new K/V vectors are quantised to int4 as they are produced and
 * attention is evaluated on the compressed representation, with no
 * dequantised fp16 K/V ever written to memory ("Open-TQ-Metal: Fused
 * Compressed-Domain Attention for Long-Context LLM Inference on Apple
 * Silicon", arXiv 2604.16957, abstract; zingnex Open-TQ-Metal page, sections
 * on on-the-fly quantisation, compressed-domain attention and eliminating
 * intermediate matrices).  The quantiser is symmetric group abs-max with
 * nibble packing, optionally after a sign-randomised Hadamard rotation
 * ("SRFT + int4 KV-cache", agents-report page, core-method section; AdapTQ,
 * zingnex page, section on Fast Hadamard Rotation).  The call shape follows
 * AdapTQ's engine API (section on the native Python API): a fixed-capacity
 * cache, an append of new K/V, and an attention call over the cache.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing.  Its only state is one device word per GPU (set up
 *    by the first call on that GPU) that collects device-side contract
 *    violations for otq_last_device_error.
 *  - Descriptor structs (otq_cache, otq_plan) live in HOST memory and are
 *    read during the call only.
 *  - `stream` is a hipStream_t (NULL = the default stream) of the current
 *    device.  Work is enqueued asynchronously; the return value reports only
 *    what the host can check (arguments) and launch failures.
 *  - Device-side preconditions (positions and lengths inside the cache) are
 *    the caller's contract.  A kernel that meets a value outside it clamps or
 *    skips as documented per call, never touches memory outside the cache,
 *    and records the violation for otq_last_device_error.
 *  - No entry point throws; all return an otq_status (0 = OTQ_OK).
 *  - Argument errors are detected on the host before any HIP call is made.
 */
#ifndef OTQ_H
#define OTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OTQ_ABI_VERSION 8

/* Elements per quantisation group (one fp32 scale each), along head_dim. */
#define OTQ_GROUP 32
/* Tokens per tile of the V code layout; capacity must be a multiple. */
#define OTQ_TILE 32

typedef enum otq_status {
    OTQ_OK = 0,
    OTQ_EINVAL = -1,       /* null pointer, bad count, Hq % Hkv != 0, ...      */
    OTQ_ECAPACITY = -2,    /* max_len or n_new larger than the cache capacity */
    OTQ_EUNSUPPORTED = -3, /* head_dim not in {64,128,192,256}, bad dtype, G>16 */
    OTQ_EWORKSPACE = -4,   /* workspace null or smaller than required          */
    OTQ_EDEVICE = -5       /* a HIP launch failed                              */
} otq_status;

typedef enum otq_dtype { OTQ_F16 = 0, OTQ_BF16 = 1 } otq_dtype;

/* The kind of the cache's rotations (otq_cache.rot_kind): K's when
 * k_rot_signs != NULL, V's when v_rot_signs != NULL. */
typedef enum otq_rot_kind {
    OTQ_ROT_SRHT = 0, /* sign-randomised Walsh-Hadamard transform */
    OTQ_ROT_SRFT = 1  /* sign-randomised FFT                      */
} otq_rot_kind;

/*
 * A quantised KV cache for one attention layer: caller-owned device arrays,
 * described by a host struct.
 *
 * Quantisation (per vector x of head_dim elements, per group g of 32
 * consecutive elements, all in IEEE fp32 with round-half-to-even):
 *     s_g  = max_i |x_i| / 7
 *     c_i  = 0 if s_g == 0, else clamp(rint(x_i / s_g), -8, 7)
 * K only, when k_rot_signs != NULL, x is first replaced by
 *     y = rot_norm * H (k_rot_signs (.) x)
 * with H the Sylvester-ordered Walsh-Hadamard matrix, evaluated as in-place
 * butterflies (a + b, a - b) in ascending stride order, then one multiply by
 * rot_norm (pass fp32(1/sqrt(head_dim))).  That is rot_kind = OTQ_ROT_SRHT.
 * With rot_kind = OTQ_ROT_SRFT ("SRFT + int4 KV-cache" page, core-method
 * section: a sign-randomised FFT in place of the Hadamard rotation) the D
 * reals are instead D/2 complex numbers z_j = (x_2j, x_2j+1), signs applied
 * to the reals first, transformed by the radix-2 decimation-in-frequency FFT
 * in place: stages of half-size h = N/2, ..., 1 (N = D/2) replace (z_j,
 * z_j+h) with (z_j + z_j+h, (z_j - z_j+h) W^t), W = exp(-2 pi i / N), t = (j
 * mod h) N / (2h), which leaves DFT coefficient bitrev(k) at position k;
 * then one multiply by rot_norm (pass fp32(1/sqrt(head_dim / 2))).  Each
 * step is one fp32 operation, the complex product (dr wr - di wi, dr wi +
 * di wr) with products rounded before the sum, and the twiddles (wr, wi)
 * are the correctly rounded fp32 cos and -sin of 2 pi t / N.
 * head_dim 192 (N = 96 = 3 * 32; int4 codes only, K rotated by the FFT kind
 * only, V not rotated, no fused append) takes the mixed-radix form of the
 * same FFT ("SRFT + int4 KV-cache" page, core method: mixed radix for widths
 * that are not powers of two): first a radix-3 stage, output position
 * 32 m + j (m = 0, 1, 2; j < 32) from a_i = z_j+32i with u = a_0 - 0.5 (a_1 +
 * a_2) and t = fp32(sqrt(3)/2) (a_1 - a_2): a_0 + a_1 + a_2, (u - i t) W^j
 * and (u + i t) W^2j; then, inside each block of 32, the radix-2 stages of
 * half-size h = 16, ..., 1 as above with t = (j mod h) 96 / (2h); W =
 * exp(-2 pi i / 96); rot_norm = fp32(1/sqrt(96)).
 * The query is rotated the same way inside otq_sdpa_int4_decode, so scores
 * are unchanged by the rotation.
 * K only, when k_chan_scale != NULL (a per-coordinate scale lambda applied
 * after the rotation and before the group abs-max: "SRFT + int4 KV-cache"
 * page, core-method section), x (rotated or not) is then replaced by
 *     z_i = x_i * k_chan_scale[i]      (one fp32 multiply)
 * and attention reads K^_i = code_i * s_g / k_chan_scale[i]: the query is
 * divided by the scale inside otq_sdpa_int4_decode.
 * V, when v_rot_signs != NULL, is rotated before quantisation exactly as K
 * would be (its own signs, the same rot_kind and rot_norm), and the
 * attention output is brought back to the original basis by the inverse of
 * that rotation: out <- v_rot_signs (.) (rot_norm * H out) for the Hadamard
 * kind; for the FFT kind the stages undone in reverse order (half-size 1,
 * 2, ..., N/2; a pair (a', b') becomes (a' + b' conj(W^t), a' - b'
 * conj(W^t))), then rot_norm and the signs.
 *
 * Layouts (B = batch, H = num_kv_heads, D = head_dim, C = capacity):
 *  Codes are two's-complement int4 nibbles; a byte holds an even channel in
 *  its low nibble and the next channel in its high nibble.
 *  k_codes  uint8 [B][H][C][D/2]: a token's row is D/8 32-bit words; with
 *           NG = D/32 groups, word (r*NG + g), r = 0..3, holds channels
 *           32g + 8r .. 32g + 8r + 7, channel 32g + 8r + k in nibble k
 *           (byte k/2, low nibble for even k).  So row quarter r (bytes
 *           [r*D/8, (r+1)*D/8)) carries 8 channels of every group.
 *  k_scales float [B][H][C][D/32], v_scales likewise: s_g per token, group.
 *  v_codes  uint8 [B][H][C/32][16*D]: regrouped per tile of 32 tokens so
 *           that each 32-bit word holds 8 tokens of one channel.  For tile-relative token u
 *           (0..31) let quarter r = (u % 16) / 4 and slot j = 4*(u / 16) +
 *           (u % 4).  Channel c with cb = c / 16, n = c % 16, a = cb / 4,
 *           b = cb % 4 owns word ((a*4 + r)*16 + n)*4 + b of the tile, and
 *           slot j sits in byte j/2 of that word, low nibble for even j.
 *           Tokens 2m and 2m+1 always share a byte.
 *
 * Bytes per array: codes B*H*C*D/2, scales B*H*C*(D/32)*4.
 *
 * 2- and 3-bit codes (code_bits = 2 or 3; AdapTQ page, core mechanisms: 2-,
 * 3- and 4-bit quantisation): s_g = max_i |x_i| / (2^(b-1) - 1) and c_i =
 * clamp(rint(x_i / s_g), -2^(b-1), 2^(b-1) - 1), otherwise as above; fields
 * are the codes' two's complement b bits.
 *  k_codes  uint8 [B][H][C][D*b/8]: plain little-endian bit-stream rows,
 *           element i at bits [b i, b i + b) of the row.
 *  v_codes  uint8 [B][H][C/32][32*D*b/8]: per tile of 32 tokens, read as
 *           32-bit words (little-endian).  For tile-relative token u let
 *           h = u / 16, r = (u % 16) / 4, m = u % 4; for channel c let
 *           cb = c / 16, n = c % 16, l = 16 r + n.
 *           b = 2: the field of (u, c) is at bit 16 h + 8 (cb % 2) + 2 m of
 *                  word l (D/32) + cb / 2.
 *           b = 3: with qd = cb / 4 and w = cb % 4, for w < 3 the field is at
 *                  bit 16 h + 3 m of word l (3D/64) + 3 qd + w; for w = 3,
 *                  bit i (0..2) of the field is at bit 16 h + 12 + p % 4 of
 *                  word l (3D/64) + 3 qd + p / 4, p = 3 m + i.
 *  scales as above.  Rotations and the per-channel scale apply as for int4.
 * Split passes: b-bit caches whose K is neither rotated nor channel-scaled
 * take the MFMA variant (the default; any G <= 16), the others the vector
 * variant (any G <= 16; OTQ_EUNSUPPORTED if MFMA is forced).
 * otq_sdpa_int4_decode_append takes these caches too: its combine quantises
 * the new token with the b-bit rule, writes its K row whole and sets its V
 * fields in their tile.
 */
typedef struct otq_cache {
    int32_t batch;
    int32_t num_kv_heads;
    int32_t head_dim;      /* 64, 128, 256, or 192 (int4 codes, see above) */
    int32_t capacity;      /* tokens per sequence, multiple of OTQ_TILE, >= 32 */
    uint8_t *k_codes;
    float *k_scales;
    uint8_t *v_codes;
    float *v_scales;
    const float *k_rot_signs; /* device [D] of +1.0f / -1.0f, 16-byte aligned, or NULL */
    float rot_norm;           /* used only when k_rot_signs or v_rot_signs != NULL */
    const float *k_chan_scale; /* device [D] fp32 lambda, finite and > 0, 16-byte aligned, or NULL */
    const float *v_rot_signs;  /* device [D] of +1.0f / -1.0f, 16-byte aligned, or NULL */
    int32_t rot_kind;          /* otq_rot_kind of both rotations; read only when
                                  k_rot_signs or v_rot_signs != NULL */
    int32_t code_bits;         /* 4 (or 0) for the int4 layouts above; 2 or 3 for b-bit codes */
} otq_cache;

/* Human-readable name of a status code (static string). */
const char *otq_status_str(int status);

/* OTQ_ABI_VERSION of the loaded library. */
int otq_abi_version(void);

/*
 * Byte sizes of one codes array and one scales array of a cache with these
 * dimensions and code width (code_bits 4 or 0 for int4, 2 or 3; K and V
 * have the same sizes): codes B*H*C*D*code_bits/8, scales B*H*C*(D/32)*4.
 * Returns OTQ_OK, or OTQ_EINVAL / OTQ_EUNSUPPORTED for dimensions or a code
 * width the cache does not support.  Pure host arithmetic.
 */
int otq_cache_array_bytes(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                          int32_t capacity, int32_t code_bits, size_t *codes_bytes,
                          size_t *scales_bytes);

/* Total bytes of the four arrays (0 for unsupported dimensions). */
size_t otq_cache_bytes(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                       int32_t capacity, int32_t code_bits);

/*
 * Measurement aid, not a step of the method: read every byte of buf once
 * with non-temporal 16-byte loads (as the split pass reads the cache), over
 * `blocks` workgroups of 256 threads, and write one word per workgroup into
 * sink (device uint32 [blocks]).  Timing it gives the streaming-read rate the
 * decode kernels' bandwidth is compared with.  buf: device, 16-byte aligned,
 * bytes a nonzero multiple of 16.  Returns OTQ_OK, OTQ_EINVAL or OTQ_EDEVICE.
 */
int otq_stream_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks, void *stream);

/* Bits of the device error word (otq_last_device_error). */
#define OTQ_DEVERR_POS 1u  /* otq_quantize_append met pos[b] < 0 or pos[b] + n_new > capacity
                              (the tokens outside [0, capacity) were skipped) */
#define OTQ_DEVERR_LENS 2u /* a decode call met lens[b] < 0 or lens[b] > max_len
                              (it was clamped to [0, max_len]) */

/*
 * The device-side contract violations (a bit-or of OTQ_DEVERR_*) recorded on
 * the current device since the previous call, which clears them.  The word
 * is read and cleared in one atomic step on `stream` after the work queued
 * before it; the call then waits for the stream.  Returns OTQ_OK, OTQ_EINVAL
 * (flags NULL) or OTQ_EDEVICE.  The word is shared by every call on the
 * device, whatever its stream.
 */
int otq_last_device_error(void *stream, uint32_t *flags);

/*
 * Quantise n_new new K and V vectors per (sequence, KV head) and store them
 * into the cache at token positions pos[b] + t, t = 0..n_new-1 (Open-TQ-Metal
 * abstract: the cache is quantised to int4 on the fly).
 *
 *  k, v   device [B][H][n_new][D] fp16 or bf16 (dtype), contiguous and
 *         16-byte aligned (read 8 channels at a time).
 *  pos    device int32 [B].  Contract: 0 <= pos[b] and
 *         pos[b] + n_new <= capacity.  Tokens that fall outside
 *         [0, capacity) are skipped (never written out of bounds), and the
 *         violation sets OTQ_DEVERR_POS.
 *  Codes and scales of every token not in the range are left untouched,
 *  including the neighbour that shares a V byte with a new token.
 *  Host errors: OTQ_EINVAL (null pointer, misaligned k or v, n_new < 1, a
 *  misaligned per-channel vector or an unknown rot_kind in the descriptor),
 *  OTQ_EUNSUPPORTED (head_dim, dtype), OTQ_ECAPACITY (n_new > capacity).
 */
int otq_quantize_append(const void *k, const void *v, int32_t dtype, int32_t n_new,
                        const otq_cache *cache, const int32_t *pos, void *stream);

/* Kernel variants of the split pass. */
typedef enum otq_variant {
    OTQ_VARIANT_AUTO = 0,
    OTQ_VARIANT_VECTOR = 1, /* fp32 vector FMA, G in {1, 2, 4} (not G = 4 at D = 256) */
    OTQ_VARIANT_MFMA = 2    /* fp16 MFMA 16x16x32, any G <= 16; the default */
} otq_variant;

/*
 * Work split of one decode call (flash-decoding style): the token axis of
 * every (sequence, KV head) is cut into pieces of `chunk` tokens; split s
 * takes pieces s, s + S, s + 2S, ... (S = num_splits) and is one workgroup
 * producing an unnormalised partial (m, l, o) over them, and a second kernel
 * merges the partials of each (sequence, query head).  When S * chunk >=
 * max_len every split has one contiguous piece; otherwise the pieces of a
 * head's splits interleave, so that the splits read one compact window of
 * the cache at a time (the MFMA variant on a single sequence only).
 */
typedef struct otq_plan {
    int32_t chunk;       /* tokens per piece, multiple of 128 */
    int32_t num_splits;  /* workgroups per (sequence, KV-head group), >= 1 */
    int32_t variant;     /* OTQ_VARIANT_VECTOR or OTQ_VARIANT_MFMA */
    int32_t reserved;
    size_t workspace_bytes;
} otq_plan;

/*
 * Choose the plan for a decode call.  chunk_override = 0,
 * variant_override = OTQ_VARIANT_AUTO and splits_override = 0 pick defaults
 * from the shape; nonzero values force them (chunk must be a positive
 * multiple of 128).  A split count below ceil(max_len / chunk) interleaves
 * the pieces; it is honoured only where that is supported (the MFMA variant,
 * batch 1, chunk / 32 a power of two) and otherwise replaced by
 * ceil(max_len / chunk), as is any larger count.  A plan passed to a decode
 * call is re-derived the same way from its chunk, variant and num_splits for
 * the call's max_len.  Any valid plan gives the same result up to fp32
 * rounding.  Pure host arithmetic.
 */
int otq_sdpa_plan(int32_t num_q_heads, const otq_cache *cache, int32_t max_len,
                  int32_t chunk_override, int32_t variant_override, int32_t splits_override,
                  otq_plan *plan);

/* Workspace bytes otq_sdpa_int4_decode needs for the default plan (0 on error). */
size_t otq_sdpa_workspace_bytes(int32_t num_q_heads, const otq_cache *cache, int32_t max_len);

/*
 * Decode attention on the packed cache (Open-TQ-Metal abstract: attention
 * computed directly on the compressed representation; zingnex page, section
 * on compressed-domain attention):
 *
 *   out[b,h] = sum_t w_t V^[b,kv(h),t] / sum_t w_t,  t < lens[b]
 *   w_t      = exp(S_t - max_u S_u),  S_t = scale * q'[b,h] . K^[b,kv(h),t]
 *
 * with K^ = code * s (V^ likewise), kv(h) = h / (num_q_heads / H), q' = q
 * rotated as K was when cache->k_rot_signs != NULL.  lens[b] == 0 gives 0.
 *
 *  q        device [B][Hq][D] fp16/bf16 (dtype), 16-byte aligned; any finite
 *           values (the MFMA variant scales each row by a power of two
 *           before its fp16 products).
 *  lens     device int32 [B]; values are clamped to [0, max_len] (a value
 *           outside sets OTQ_DEVERR_LENS).  Cache slots at or past lens[b]
 *           are never read into the result, whatever they hold.
 *  max_len  host bound on lens, 1..capacity; sizes the split grid.
 *  out      device fp32 [B][Hq][D], 16-byte aligned.
 *  workspace device scratch of at least otq_sdpa_workspace_bytes(...) bytes
 *           (or plan->workspace_bytes); contents need no initialisation.
 * Host errors: OTQ_EINVAL (null or misaligned pointers, Hq % H != 0, a
 * non-finite scale), OTQ_EUNSUPPORTED (head_dim, dtype, G > 16, or a forced
 * variant that does not support G), OTQ_ECAPACITY (max_len > capacity),
 * OTQ_EWORKSPACE.
 *
 * Value range of the MFMA variant: the value operand p * s_v * 2^E is kept
 * inside fp16's range by a power of two E that follows the largest V scale
 * seen (over the whole fp32 range of scales), so V of any finite magnitude
 * keeps full precision.
 */
int otq_sdpa_int4_decode(const void *q, int32_t dtype, int32_t num_q_heads,
                         const otq_cache *cache, const int32_t *lens, int32_t max_len,
                         float scale, float *out, void *workspace, size_t workspace_bytes,
                         void *stream);

/* The same call with an explicit plan from otq_sdpa_plan (for tuning and
 * split-invariance checks). */
int otq_sdpa_int4_decode_planned(const void *q, int32_t dtype, int32_t num_q_heads,
                                 const otq_cache *cache, const int32_t *lens,
                                 int32_t max_len, float scale, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 const otq_plan *plan, void *stream);

/*
 * One decode step: quantise the new token of every sequence into the cache
 * at position lens[b] - 1 (as otq_quantize_append with n_new = 1 and
 * pos = lens[b] - 1 would), and attend over tokens [0, lens[b]) as
 * otq_sdpa_int4_decode does, with no separate append launch.  The token is
 * quantised on the fly as it is produced and attention reads only the
 * compressed form (Open-TQ-Metal abstract; zingnex page, sections on
 * on-the-fly quantisation and compressed-domain attention): the split pass
 * covers the cached tokens [0, lens[b] - 1), and the combine pass quantises
 * the new token, writes it and merges it as one more term.
 *
 *  k_new, v_new  device [B][Hkv][D] fp16/bf16 (dtype): the new token's K, V.
 *  plan          from otq_sdpa_plan, or NULL for the default plan.
 * Sequences with lens[b] == 0 append nothing and get zeros.  lens[b] is
 * clamped to [0, max_len] before anything else, by every kernel of the
 * call alike (so lens[b] > max_len appends at max_len - 1).  Other
 * arguments, contracts and errors as for otq_sdpa_int4_decode_planned; the
 * cache must hold tokens [0, lens[b] - 1) already.
 * At head_dim 192 the combine transforms the new token's rotated K with the
 * mixed-radix FFT described above, in every channel slice of a row.
 */
int otq_sdpa_int4_decode_append(const void *q, const void *k_new, const void *v_new,
                                int32_t dtype, int32_t num_q_heads, const otq_cache *cache,
                                const int32_t *lens, int32_t max_len, float scale, float *out,
                                void *workspace, size_t workspace_bytes,
                                const otq_plan *plan, void *stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): otq_sdpa_int4_decode_append
 * with its workspace in a fixed array of OTQ_NOALLOC_SCRATCH_BYTES bytes that
 * the library keeps on each GPU (set up on the first call on that GPU and
 * held until the process ends).  The call itself allocates nothing.
 *
 *  Arguments, results and errors as for otq_sdpa_int4_decode_append, except
 *  OTQ_EWORKSPACE when the plan's workspace_bytes exceeds
 *  OTQ_NOALLOC_SCRATCH_BYTES (checked on the host), and OTQ_EDEVICE when the
 *  array's address cannot be obtained.
 *  Every call on one GPU shares that GPU's array: calls that overlap on one
 *  GPU (other streams, other host threads) race and must be serialised by
 *  the caller.  The array needs no clearing between calls (the split pass
 *  writes every partial the combine reads).
 */
#define OTQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int otq_sdpa_int4_decode_append_noalloc(const void *q, const void *k_new, const void *v_new,
                                        int32_t dtype, int32_t num_q_heads,
                                        const otq_cache *cache, const int32_t *lens,
                                        int32_t max_len, float scale, float *out,
                                        const otq_plan *plan, void *stream);

/*
 * The two phases of otq_sdpa_int4_decode as separate calls, for callers
 * that time them apart or merge partials computed elsewhere (each split of
 * the token axis is independent until the combine).
 *
 * otq_sdpa_int4_split writes the partials of every non-empty split into the
 * workspace, laid out as
 *   part_o  fp32 [B][Hq][num_splits][D]      at byte offset 0
 *   part_ml fp32 [B][Hq][num_splits][2]      at byte offset
 *           round_up(B*Hq*num_splits*D*4, 256)
 * where split s covers tokens [s*chunk, min((s+1)*chunk, lens[b])), m is the
 * split's reference in log2 units (score * log2(e)), l = sum 2^(S*log2e - m)
 * and o = sum 2^(S*log2e - m) V^; the kernel chooses m (near the largest
 * score, shifted by a power of two that keeps o in range) and any m gives
 * the same merged result.
 * Splits with s*chunk >= lens[b] are not
 * written.  otq_sdpa_lse_combine merges the first ceil(lens[b]/chunk)
 * partials of each row into out.  Arguments and errors as for
 * otq_sdpa_int4_decode_planned.  With cache->v_rot_signs set, V^ and so
 * part_o are in V's rotated basis; otq_sdpa_lse_combine then applies the
 * inverse rotation to out (one block per output row).
 *
 * For a batch of 2..256 sequences the split pass is two launches: a
 * one-workgroup kernel first writes, at byte offset
 * round_up(part_ml offset + B*Hq*num_splits*8, 256) of the workspace, which
 * work item (split, sequence) each split workgroup takes, longest first
 * (the full chunks, then the last partial chunks by decreasing length), so
 * that the hardware's in-order start of workgroups balances sequences of
 * unequal length.  The partials are the same either way.
 */
int otq_sdpa_int4_split(const void *q, int32_t dtype, int32_t num_q_heads,
                        const otq_cache *cache, const int32_t *lens, int32_t max_len,
                        float scale, void *workspace, size_t workspace_bytes,
                        const otq_plan *plan, void *stream);

int otq_sdpa_lse_combine(int32_t num_q_heads, const otq_cache *cache, const int32_t *lens,
                         int32_t max_len, const void *workspace, size_t workspace_bytes,
                         const otq_plan *plan, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* OTQ_H */
