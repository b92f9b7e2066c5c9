// api.hip - the C ABI of libotq: host-side validation, planning and launch.
//
// Every argument the host can see is checked before the first HIP call, so a
// bad call returns a status and touches no device state.  Nothing here
// allocates: buffers, descriptors and the workspace belong to the caller
// (the AdapTQ page, section on zero heap allocation, keeps its hot path free
// of allocation for the same reason: predictable latency).
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/otq.h"
#include "kernels.hpp"

// The device error word of each GPU: [0] collects the kernels' contract
// violations (OTQ_DEVERR_*), [1] receives the value otq_last_device_error
// takes.  Host code uses the address hipGetSymbolAddress gives per device,
// never this name (which on the host is only a stand-in for the symbol).
static __device__ unsigned otq_device_error_word[2];

// The workspace of otq_sdpa_int4_decode_append_noalloc: one copy per GPU,
// held until the process ends.  As above, host code only ever uses the
// per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[OTQ_NOALLOC_SCRATCH_BYTES];

namespace {

// Reads and clears the live word in one atomic step.
__global__ void take_device_error_kernel(unsigned* w)
{
    w[1] = __hip_atomic_exchange(&w[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-device set-up, done once per device on the first call that launches
// work there (with that device current).
constexpr int kMaxDevices = 64;
struct DeviceState {
    std::once_flag once;
    hipError_t rc = hipSuccess;
    unsigned* err = nullptr;  // this device's otq_device_error_word
    void* scratch = nullptr;  // this device's scratch array
};
DeviceState g_devices[kMaxDevices];

// The current device's state, or null if it could not be set up.
DeviceState* device_state()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceState& d = g_devices[dev];
    std::call_once(d.once, [&d] {
        void* p = nullptr;
        d.rc = hipGetSymbolAddress(&p, HIP_SYMBOL(otq_device_error_word));
        if (d.rc != hipSuccess) return;
        d.err = static_cast<unsigned*>(p);
        p = nullptr;
        d.rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.rc != hipSuccess) return;
        d.scratch = p;
    });
    return d.rc == hipSuccess && d.err && d.scratch ? &d : nullptr;
}

// The current device's error word for a launch (null: OTQ_EDEVICE).
unsigned* error_word()
{
    DeviceState* d = device_state();
    return d ? d->err : nullptr;
}

constexpr int kChunkAlign = 128;  // 4 waves x 32-token tiles
constexpr int kMaxChunk = 8192;  // measured: larger chunks starve the grid on ragged batches
constexpr int kTargetWaves = 1024;  // split waves aimed for (one per SIMD)
constexpr int kOrderedWaveFactor = 8;  // measured on the ragged 32-sequence batch: chunk 2048 over 8192
constexpr int kMaxSplits = 16384;
bool pow2_int(long long x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(long long x)
{
    int k = 0;
    while ((1LL << (k + 1)) <= x) ++k;
    return k;
}

// Power-of-two widths take every kernel; 192 (three times 64) the wide ones.
bool pow2_dim(int D) { return D == 64 || D == 128 || D == 256; }
bool supported_dim(int D) { return pow2_dim(D) || otq::wide_supported_dim(D); }

int check_dims(int32_t B, int32_t H, int32_t D, int32_t cap)
{
    if (B < 1 || H < 1 || cap < OTQ_TILE || cap % OTQ_TILE != 0) return OTQ_EINVAL;
    if (!supported_dim(D)) return OTQ_EUNSUPPORTED;
    // element offsets are formed in 64-bit; keep each array below 2^62 bytes
    const unsigned __int128 n = (unsigned __int128)B * H * cap * D;
    if (n > ((unsigned __int128)1 << 62)) return OTQ_EINVAL;
    return OTQ_OK;
}

// Code width of a cache: 0 (a descriptor that predates the field) is int4.
int code_bits(const otq_cache* c) { return c->code_bits == 0 ? 4 : c->code_bits; }

int check_cache(const otq_cache* c)
{
    if (!c) return OTQ_EINVAL;
    const int rc = check_dims(c->batch, c->num_kv_heads, c->head_dim, c->capacity);
    if (rc != OTQ_OK) return rc;
    if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales) return OTQ_EINVAL;
    // the per-channel vectors are read 4 floats at a time
    if ((((uintptr_t)c->k_rot_signs) & 15) != 0 || (((uintptr_t)c->k_chan_scale) & 15) != 0 ||
        (((uintptr_t)c->v_rot_signs) & 15) != 0)
        return OTQ_EINVAL;
    if ((c->k_rot_signs || c->v_rot_signs) && c->rot_kind != OTQ_ROT_SRHT && c->rot_kind != OTQ_ROT_SRFT)
        return OTQ_EINVAL;
    if (c->code_bits != 0 && c->code_bits != 2 && c->code_bits != 3 && c->code_bits != 4) return OTQ_EINVAL;
    if (!pow2_dim(c->head_dim)) {
        // the wide widths: int4 codes; K rotated by the FFT kind only (the
        // Hadamard form needs a power of two); V unrotated
        if (c->code_bits != 0 && c->code_bits != 4) return OTQ_EUNSUPPORTED;
        if (c->k_rot_signs && c->rot_kind != OTQ_ROT_SRFT) return OTQ_EUNSUPPORTED;
        if (c->v_rot_signs) return OTQ_EUNSUPPORTED;
    }
    return OTQ_OK;
}

// The rotations' kind as the kernels take it (checked by check_cache).
int rot_kind(const otq_cache* c)
{
    return (c->k_rot_signs || c->v_rot_signs) && c->rot_kind == OTQ_ROT_SRFT ? 1 : 0;
}

// Batches whose split blocks take their items longest first (one sequence
// needs no order: its chunks are equal but the last).
bool ordered_batch(int32_t B) { return B > 1 && B <= otq::kOrderMaxBatch; }

// The b-bit MFMA split pass: 2- or 3-bit codes, power-of-two head_dim,
// G <= 16; a rotated or channel-scaled K (hi + lo query) up to head_dim 128;
// and int4 codes at head_dim 192 (any K the cache takes there).
bool bits_mfma_ok(const otq_cache* c, int G)
{
    return otq::split_bits_mfma_supports(c->head_dim, G, code_bits(c), c->k_rot_signs != nullptr,
                                         c->k_chan_scale != nullptr);
}

// The split pass is the b-bit matrix-core kernel: b-bit codes, or int4 at
// the wide widths.
bool takes_bits_mfma(const otq_cache* c, int variant)
{
    return variant == OTQ_VARIANT_MFMA && (code_bits(c) != 4 || !pow2_dim(c->head_dim));
}

int make_plan(int32_t Hq, const otq_cache* c, int32_t max_len, int32_t chunk_ov,
              int32_t variant_ov, int32_t splits_ov, otq_plan* p)
{
    int rc = check_cache(c);
    if (rc != OTQ_OK) return rc;
    if (!p || Hq < 1 || Hq % c->num_kv_heads != 0 || max_len < 1) return OTQ_EINVAL;
    if (max_len > c->capacity) return OTQ_ECAPACITY;
    const int G = Hq / c->num_kv_heads;
    const int D = c->head_dim;
    if (G > 16) return OTQ_EUNSUPPORTED;

    int variant = variant_ov;
    if (!pow2_dim(D)) {
        // the wide widths: the matrix-core pass by default, the vector pass
        // (any G <= 16) when asked for
        if (variant == OTQ_VARIANT_AUTO) variant = bits_mfma_ok(c, G) ? OTQ_VARIANT_MFMA : OTQ_VARIANT_VECTOR;
        if (variant == OTQ_VARIANT_MFMA && !bits_mfma_ok(c, G)) return OTQ_EUNSUPPORTED;
    } else if (variant == OTQ_VARIANT_AUTO) {
        // the MFMA variant is the faster one at every measured G (1, 2, 4, 8)
        // (2- and 3-bit codes too, on a K that is neither rotated nor channel-scaled)
        variant = code_bits(c) == 4   ? (otq::split_mfma_supports(D, G) ? OTQ_VARIANT_MFMA : OTQ_VARIANT_VECTOR)
                  : bits_mfma_ok(c, G) ? OTQ_VARIANT_MFMA
                                     : OTQ_VARIANT_VECTOR;
    }
    if (!pow2_dim(D)) {
        if (variant != OTQ_VARIANT_VECTOR && variant != OTQ_VARIANT_MFMA) return OTQ_EINVAL;
    } else if (code_bits(c) != 4) {  // the b-bit split passes: vector (any), MFMA (plain K)
        if (variant == OTQ_VARIANT_MFMA) {
            if (!bits_mfma_ok(c, G)) return OTQ_EUNSUPPORTED;
        } else if (variant != OTQ_VARIANT_VECTOR) {
            return OTQ_EINVAL;
        }
    } else if (variant == OTQ_VARIANT_VECTOR) {
        if (!otq::split_vector_supports(D, G)) return OTQ_EUNSUPPORTED;
    } else if (variant == OTQ_VARIANT_MFMA) {
        if (!otq::split_mfma_supports(D, G)) return OTQ_EUNSUPPORTED;
        // the MFMA variant addresses two heads of codes with 32-bit buffer offsets
        if ((long long)2 * c->capacity * (D / 2) >= ((long long)1 << 31)) return OTQ_EUNSUPPORTED;
    } else {
        return OTQ_EINVAL;
    }

    int chunk = chunk_ov;
    if (chunk == 0) {
        long long units = (long long)c->batch * c->num_kv_heads;
        int waves = 4, align = kChunkAlign;
        if (variant == OTQ_VARIANT_MFMA && !takes_bits_mfma(c, variant)) {
            units /= otq::split_mfma_heads_per_wave(D, G, c->num_kv_heads);
            waves = otq::split_mfma_block_waves(D);
            align = waves * OTQ_TILE;  // one tile per wave and round
        } else if (variant == OTQ_VARIANT_MFMA) {
            units /= otq::split_bits_mfma_heads_per_wave(D, G, c->num_kv_heads, c->k_rot_signs || c->k_chan_scale);
        }
        // a batch takes its items longest first, which balances unequal
        // lengths better the more (smaller) items there are
        // the vector b-bit split pass hides latency only with several blocks per CU
        const bool bits_vec = code_bits(c) != 4 && variant == OTQ_VARIANT_VECTOR;
        // the b-bit MFMA pass (one KV head per block) is measured fastest
        // with two waves per SIMD: on the 70B layer at 128K (2-bit codes),
        // 32.8 us at chunk 2048 against 37.3 us at 1024
        const bool bits_mfma = takes_bits_mfma(c, variant);
        // so is the int4 pass at head_dim 256 (one KV head per wave): on the
        // Gemma-shaped layer (16 KV heads, 64K tokens) 63.1 us at chunk 2048
        // against 63.9-64.6 us at 4096
        const bool wide_mfma = code_bits(c) == 4 && variant == OTQ_VARIANT_MFMA && D == 256;
        const long long target = (ordered_batch(c->batch) || bits_vec) ? kTargetWaves * kOrderedWaveFactor
                                 : (bits_mfma || wide_mfma)            ? kTargetWaves * 2
                                                                       : kTargetWaves;
        const long long groups = target / waves;
        long long want = ((long long)max_len * units + groups - 1) / groups;
        want = (want + align - 1) / align * align;
        if (want < kChunkAlign) want = kChunkAlign;
        if (want > kMaxChunk) want = kMaxChunk;
        chunk = (int)want;
    } else if (chunk < 0 || chunk % kChunkAlign != 0) {
        return OTQ_EINVAL;
    }
    if (splits_ov < 0) return OTQ_EINVAL;
    // interleaved pieces (several per split): the MFMA pass on one sequence
    // (a batch orders its blocks by whole chunks), 2^k tiles per piece
    const bool can_interleave = variant == OTQ_VARIANT_MFMA && pow2_dim(D) && code_bits(c) == 4 &&
                                !ordered_batch(c->batch) && pow2_int(chunk / OTQ_TILE) &&
                                chunk % OTQ_TILE == 0;
    long long S = ((long long)max_len + chunk - 1) / chunk;
    if (splits_ov != 0 && splits_ov < S && can_interleave) {
        S = splits_ov;  // the caller's split count, over interleaved pieces
    }
    if (S > kMaxSplits) return OTQ_EINVAL;  // bounds the partials' workspace
    const unsigned __int128 rows = (unsigned __int128)c->batch * Hq * S;
    const unsigned __int128 o_bytes = rows * D * sizeof(float);
    const unsigned __int128 o_aligned = (o_bytes + 255) / 256 * 256;
    const unsigned __int128 ml_aligned = (rows * 2 * sizeof(float) + 255) / 256 * 256;
    // a batch also holds the split blocks' longest-first items: (split,
    // sequence) per block, at most S * Hkv * B blocks
    const unsigned __int128 order_bytes =
        ordered_batch(c->batch) ? (unsigned __int128)S * c->num_kv_heads * c->batch * 2 * sizeof(int32_t) : 0;
    const unsigned __int128 total = o_aligned + ml_aligned + order_bytes;
    if (total > ((unsigned __int128)1 << 62)) return OTQ_EINVAL;
    p->chunk = chunk;
    p->num_splits = (int32_t)S;
    p->variant = variant;
    p->reserved = 0;
    p->workspace_bytes = (size_t)total;
    return OTQ_OK;
}

}  // namespace

extern "C" {

const char* otq_status_str(int status)
{
    switch (status) {
    case OTQ_OK: return "OTQ_OK";
    case OTQ_EINVAL: return "OTQ_EINVAL: invalid argument";
    case OTQ_ECAPACITY: return "OTQ_ECAPACITY: length exceeds cache capacity";
    case OTQ_EUNSUPPORTED: return "OTQ_EUNSUPPORTED: unsupported head_dim, dtype or head grouping";
    case OTQ_EWORKSPACE: return "OTQ_EWORKSPACE: workspace missing or too small";
    case OTQ_EDEVICE: return "OTQ_EDEVICE: HIP launch failed";
    default: return "unknown otq status";
    }
}

int otq_abi_version(void) { return OTQ_ABI_VERSION; }

int otq_cache_array_bytes(int32_t B, int32_t H, int32_t D, int32_t cap, int32_t code_bits,
                          size_t* codes_bytes, size_t* scales_bytes)
{
    const int rc = check_dims(B, H, D, cap);
    if (rc != OTQ_OK) return rc;
    const int bits = code_bits == 0 ? 4 : code_bits;
    if (bits != 2 && bits != 3 && bits != 4) return OTQ_EINVAL;
    if (bits != 4 && !pow2_dim(D)) return OTQ_EUNSUPPORTED;  // the wide widths hold int4 codes
    const size_t n = (size_t)B * H * cap;
    if (codes_bytes) *codes_bytes = n * (size_t)(D * bits / 8);
    if (scales_bytes) *scales_bytes = n * (size_t)(D / OTQ_GROUP) * sizeof(float);
    return OTQ_OK;
}

size_t otq_cache_bytes(int32_t B, int32_t H, int32_t D, int32_t cap, int32_t code_bits)
{
    size_t cb = 0, sb = 0;
    if (otq_cache_array_bytes(B, H, D, cap, code_bits, &cb, &sb) != OTQ_OK) return 0;
    return 2 * (cb + sb);
}

int otq_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream)
{
    if (!buf || !sink || blocks < 1 || bytes == 0 || bytes % 16 != 0 || (((uintptr_t)buf) & 15) != 0)
        return OTQ_EINVAL;
    return otq::launch_stream_read(buf, bytes, sink, blocks, static_cast<hipStream_t>(stream)) == hipSuccess
               ? OTQ_OK
               : OTQ_EDEVICE;
}

int otq_last_device_error(void* stream, uint32_t* flags)
{
    if (!flags) return OTQ_EINVAL;
    unsigned* w = error_word();
    if (!w) return OTQ_EDEVICE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    take_device_error_kernel<<<1, 1, 0, s>>>(w);
    if (hipGetLastError() != hipSuccess) return OTQ_EDEVICE;
    unsigned v = 0;
    if (hipMemcpyAsync(&v, w + 1, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return OTQ_EDEVICE;
    if (hipStreamSynchronize(s) != hipSuccess) return OTQ_EDEVICE;
    *flags = v;
    return OTQ_OK;
}

int otq_quantize_append(const void* k, const void* v, int32_t dtype, int32_t n_new,
                        const otq_cache* cache, const int32_t* pos, void* stream)
{
    const int rc = check_cache(cache);
    if (rc != OTQ_OK) return rc;
    if (!k || !v || !pos || n_new < 1) return OTQ_EINVAL;
    // the kernel reads 8 channels per 16-byte load
    if ((((uintptr_t)k) & 15) != 0 || (((uintptr_t)v) & 15) != 0) return OTQ_EINVAL;
    if (dtype != OTQ_F16 && dtype != OTQ_BF16) return OTQ_EUNSUPPORTED;
    if (n_new > cache->capacity) return OTQ_ECAPACITY;
    unsigned* err = error_word();
    if (!err) return OTQ_EDEVICE;
    if (!pow2_dim(cache->head_dim)) {
        const hipError_t e = otq::launch_quantize_wide(
            k, v, dtype, n_new, cache->batch, cache->num_kv_heads, cache->head_dim, cache->capacity,
            cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales, cache->k_rot_signs,
            cache->rot_norm, cache->k_chan_scale, cache->v_rot_signs, pos, err, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? OTQ_OK : OTQ_EDEVICE;
    }
    if (code_bits(cache) != 4) {
        const hipError_t e = otq::launch_quantize_bits(
            k, v, dtype, n_new, cache->batch, cache->num_kv_heads, cache->head_dim, cache->capacity,
            code_bits(cache), cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales, pos,
            otq::BitsRot{cache->k_rot_signs, cache->rot_norm, rot_kind(cache), cache->k_chan_scale,
                         cache->v_rot_signs},
            err, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? OTQ_OK : OTQ_EDEVICE;
    }
    const hipError_t e = otq::launch_quantize_append(
        k, v, dtype, n_new, cache->batch, cache->num_kv_heads, cache->head_dim, cache->capacity,
        cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales, cache->k_rot_signs,
        cache->rot_norm, rot_kind(cache), cache->k_chan_scale, cache->v_rot_signs, pos, err,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? OTQ_OK : OTQ_EDEVICE;
}

int otq_sdpa_plan(int32_t num_q_heads, const otq_cache* cache, int32_t max_len,
                  int32_t chunk_override, int32_t variant_override, int32_t splits_override,
                  otq_plan* plan)
{
    return make_plan(num_q_heads, cache, max_len, chunk_override, variant_override, splits_override, plan);
}

size_t otq_sdpa_workspace_bytes(int32_t num_q_heads, const otq_cache* cache, int32_t max_len)
{
    otq_plan p;
    if (make_plan(num_q_heads, cache, max_len, 0, OTQ_VARIANT_AUTO, 0, &p) != OTQ_OK) return 0;
    return p.workspace_bytes;
}

}  // extern "C"

namespace {

int check_workspace(const void* workspace, size_t workspace_bytes, const otq_plan& p)
{
    if (!workspace || workspace_bytes < p.workspace_bytes) return OTQ_EWORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return OTQ_EWORKSPACE;
    return OTQ_OK;
}

size_t ml_offset(const otq_cache* c, int32_t Hq, const otq_plan& p)
{
    const size_t rows = (size_t)c->batch * Hq * p.num_splits;
    return (rows * c->head_dim * sizeof(float) + 255) / 256 * 256;
}

size_t order_offset(const otq_cache* c, int32_t Hq, const otq_plan& p)
{
    const size_t rows = (size_t)c->batch * Hq * p.num_splits;
    return ml_offset(c, Hq, p) + (rows * 2 * sizeof(float) + 255) / 256 * 256;
}

// Validates a caller plan against the shape; on success *chk is the plan.
int check_plan(int32_t Hq, const otq_cache* c, int32_t max_len, const otq_plan* plan,
               otq_plan* chk)
{
    if (!plan) return OTQ_EINVAL;
    return make_plan(Hq, c, max_len, plan->chunk, plan->variant, plan->num_splits, chk);
}

int run_split(const void* q, int32_t dtype, int32_t num_q_heads, const otq_cache* cache,
              const int32_t* lens, int32_t max_len, float scale, void* workspace,
              const otq_plan& chk, hipStream_t s, int lens_offset = 0)
{
    const int D = cache->head_dim;
    otq::SplitArgs a;
    a.q = q;
    a.dtype = dtype;
    a.B = cache->batch;
    a.Hq = num_q_heads;
    a.H = cache->num_kv_heads;
    a.D = D;
    a.cap = cache->capacity;
    a.kc = cache->k_codes;
    a.ks = cache->k_scales;
    a.vc = cache->v_codes;
    a.vs = cache->v_scales;
    a.signs = cache->k_rot_signs;
    a.rot_norm = cache->rot_norm;
    a.rot_kind = rot_kind(cache);
    a.lam = cache->k_chan_scale;
    a.lens = lens;
    a.max_len = max_len;
    a.qscale = scale * otq::kLog2eHost;
    a.chunk = chk.chunk;
    a.num_splits = chk.num_splits;
    a.piece_stride = chk.chunk * chk.num_splits;
    a.piece_shift = (long long)chk.chunk * chk.num_splits >= max_len ? 30 : ilog2(chk.chunk / OTQ_TILE);
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                          ml_offset(cache, num_q_heads, chk));
    a.lens_offset = lens_offset;
    a.items = nullptr;
    a.err = error_word();
    if (!a.err) return OTQ_EDEVICE;
    if (ordered_batch(a.B)) {
        const int G = num_q_heads / a.H;
        const int groups = chk.variant != OTQ_VARIANT_MFMA ? a.H
                           : !takes_bits_mfma(cache, chk.variant)
                               ? a.H / otq::split_mfma_heads_per_wave(D, G, a.H)
                               : a.H / otq::split_bits_mfma_heads_per_wave(D, G, a.H, a.signs || a.lam);
        int2* items = reinterpret_cast<int2*>(static_cast<char*>(workspace) +
                                              order_offset(cache, num_q_heads, chk));
        if (otq::launch_split_order(lens, lens_offset, max_len, chk.chunk, chk.num_splits, groups, a.B,
                                    items, a.err, s) != hipSuccess)
            return OTQ_EDEVICE;
        a.items = items;
    }
    const hipError_t e = takes_bits_mfma(cache, chk.variant) ? otq::launch_split_bits_mfma(a, code_bits(cache), s)
                         : !pow2_dim(D)                      ? otq::launch_split_wide(a, s)
                         : code_bits(cache) != 4 ? (chk.variant == OTQ_VARIANT_MFMA
                                                        ? otq::launch_split_bits_mfma(a, code_bits(cache), s)
                                                        : otq::launch_split_bits(a, code_bits(cache), s))
                         : chk.variant == OTQ_VARIANT_MFMA ? otq::launch_split_mfma(a, s)
                                                           : otq::launch_split_vector(a, s);
    return e == hipSuccess ? OTQ_OK : OTQ_EDEVICE;
}

int run_combine(int32_t num_q_heads, const otq_cache* cache, const int32_t* lens,
                int32_t max_len, const void* workspace, const otq_plan& chk, float* out,
                hipStream_t s, const void* q = nullptr, const void* k_new = nullptr,
                const void* v_new = nullptr, int32_t dtype = 0, float scale = 0.0f)
{
    otq::CombineArgs a{};
    a.part_o = static_cast<const float*>(workspace);
    a.part_ml = reinterpret_cast<const float2*>(static_cast<const char*>(workspace) +
                                                ml_offset(cache, num_q_heads, chk));
    a.lens = lens;
    a.max_len = max_len;
    a.chunk = chk.chunk;
    a.S = chk.num_splits;
    a.B = cache->batch;
    a.Hq = num_q_heads;
    a.D = cache->head_dim;
    a.out = out;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.q = q;
    a.dtype = dtype;
    a.H = cache->num_kv_heads;
    a.cap = cache->capacity;
    a.kc = cache->k_codes;
    a.ks = cache->k_scales;
    a.vc = cache->v_codes;
    a.vs = cache->v_scales;
    a.signs = cache->k_rot_signs;
    a.rot_norm = cache->rot_norm;
    a.rot_kind = rot_kind(cache);
    a.lam = cache->k_chan_scale;
    a.vsigns = cache->v_rot_signs;
    a.qscale = scale * otq::kLog2eHost;
    a.bits = code_bits(cache);
    a.err = error_word();
    if (!a.err) return OTQ_EDEVICE;
    const hipError_t e = otq::launch_lse_combine(a, s);
    return e == hipSuccess ? OTQ_OK : OTQ_EDEVICE;
}

bool finite(float x) { return x == x && x != __builtin_huge_valf() && x != -__builtin_huge_valf(); }

// q is read 8 elements (16 bytes) at a time and out written 4 floats at a time.
bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

}  // namespace

extern "C" {

int otq_sdpa_int4_split(const void* q, int32_t dtype, int32_t num_q_heads, const otq_cache* cache,
                        const int32_t* lens, int32_t max_len, float scale, void* workspace,
                        size_t workspace_bytes, const otq_plan* plan, void* stream)
{
    otq_plan chk;
    int rc = check_plan(num_q_heads, cache, max_len, plan, &chk);
    if (rc != OTQ_OK) return rc;
    if (!q || !lens || !aligned16(q)) return OTQ_EINVAL;
    if (dtype != OTQ_F16 && dtype != OTQ_BF16) return OTQ_EUNSUPPORTED;
    if (!finite(scale)) return OTQ_EINVAL;
    if ((rc = check_workspace(workspace, workspace_bytes, chk)) != OTQ_OK) return rc;
    return run_split(q, dtype, num_q_heads, cache, lens, max_len, scale, workspace, chk,
                     static_cast<hipStream_t>(stream));
}

int otq_sdpa_lse_combine(int32_t num_q_heads, const otq_cache* cache, const int32_t* lens,
                         int32_t max_len, const void* workspace, size_t workspace_bytes,
                         const otq_plan* plan, float* out, void* stream)
{
    otq_plan chk;
    int rc = check_plan(num_q_heads, cache, max_len, plan, &chk);
    if (rc != OTQ_OK) return rc;
    if (!lens || !out || !aligned16(out)) return OTQ_EINVAL;
    if ((rc = check_workspace(workspace, workspace_bytes, chk)) != OTQ_OK) return rc;
    return run_combine(num_q_heads, cache, lens, max_len, workspace, chk, out,
                       static_cast<hipStream_t>(stream));
}

int otq_sdpa_int4_decode_planned(const void* q, int32_t dtype, int32_t num_q_heads,
                                 const otq_cache* cache, const int32_t* lens, int32_t max_len,
                                 float scale, float* out, void* workspace, size_t workspace_bytes,
                                 const otq_plan* plan, void* stream)
{
    otq_plan chk;
    int rc = check_plan(num_q_heads, cache, max_len, plan, &chk);
    if (rc != OTQ_OK) return rc;
    if (!q || !lens || !out || !aligned16(q) || !aligned16(out)) return OTQ_EINVAL;
    if (dtype != OTQ_F16 && dtype != OTQ_BF16) return OTQ_EUNSUPPORTED;
    if (!finite(scale)) return OTQ_EINVAL;
    if ((rc = check_workspace(workspace, workspace_bytes, chk)) != OTQ_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = run_split(q, dtype, num_q_heads, cache, lens, max_len, scale, workspace, chk, s);
    if (rc != OTQ_OK) return rc;
    return run_combine(num_q_heads, cache, lens, max_len, workspace, chk, out, s);
}

}  // extern "C"

namespace {

// The host checks of the fused decode step, but for the workspace; on
// success *chk is the plan to run.
int check_decode_append(const void* q, const void* k_new, const void* v_new, int32_t dtype,
                        int32_t num_q_heads, const otq_cache* cache, const int32_t* lens, int32_t max_len,
                        float scale, const float* out, const otq_plan* plan, otq_plan* chk)
{
    const int rc = plan ? check_plan(num_q_heads, cache, max_len, plan, chk)
                        : make_plan(num_q_heads, cache, max_len, 0, OTQ_VARIANT_AUTO, 0, chk);
    if (rc != OTQ_OK) return rc;
    if (!q || !k_new || !v_new || !lens || !out || !aligned16(q) || !aligned16(out)) return OTQ_EINVAL;
    if (dtype != OTQ_F16 && dtype != OTQ_BF16) return OTQ_EUNSUPPORTED;
    if (!finite(scale)) return OTQ_EINVAL;
    return OTQ_OK;
}

}  // namespace

extern "C" {

int otq_sdpa_int4_decode_append(const void* q, const void* k_new, const void* v_new, int32_t dtype,
                                int32_t num_q_heads, const otq_cache* cache, const int32_t* lens,
                                int32_t max_len, float scale, float* out, void* workspace,
                                size_t workspace_bytes, const otq_plan* plan, void* stream)
{
    otq_plan chk;
    int rc = check_decode_append(q, k_new, v_new, dtype, num_q_heads, cache, lens, max_len, scale, out,
                                 plan, &chk);
    if (rc != OTQ_OK) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, chk)) != OTQ_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = run_split(q, dtype, num_q_heads, cache, lens, max_len, scale, workspace, chk, s, 1);
    if (rc != OTQ_OK) return rc;
    return run_combine(num_q_heads, cache, lens, max_len, workspace, chk, out, s, q, k_new, v_new,
                       dtype, scale);
}

int otq_sdpa_int4_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                        int32_t dtype, int32_t num_q_heads, const otq_cache* cache,
                                        const int32_t* lens, int32_t max_len, float scale, float* out,
                                        const otq_plan* plan, void* stream)
{
    otq_plan chk;
    const int rc = check_decode_append(q, k_new, v_new, dtype, num_q_heads, cache, lens, max_len, scale,
                                       out, plan, &chk);
    if (rc != OTQ_OK) return rc;
    if (chk.workspace_bytes > OTQ_NOALLOC_SCRATCH_BYTES) return OTQ_EWORKSPACE;
    DeviceState* d = device_state();
    if (!d) return OTQ_EDEVICE;
    // the same kernels as the caller-workspace call, on this device's array
    return otq_sdpa_int4_decode_append(q, k_new, v_new, dtype, num_q_heads, cache, lens, max_len, scale,
                                       out, d->scratch, OTQ_NOALLOC_SCRATCH_BYTES, &chk, stream);
}

int otq_sdpa_int4_decode(const void* q, int32_t dtype, int32_t num_q_heads,
                         const otq_cache* cache, const int32_t* lens, int32_t max_len,
                         float scale, float* out, void* workspace, size_t workspace_bytes,
                         void* stream)
{
    otq_plan p;
    const int rc = make_plan(num_q_heads, cache, max_len, 0, OTQ_VARIANT_AUTO, 0, &p);
    if (rc != OTQ_OK) return rc;
    return otq_sdpa_int4_decode_planned(q, dtype, num_q_heads, cache, lens, max_len, scale, out,
                                        workspace, workspace_bytes, &p, stream);
}

}  // extern "C"
