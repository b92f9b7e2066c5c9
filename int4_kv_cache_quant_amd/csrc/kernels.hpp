// kernels.hpp - internal launchers of the gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace otq {

constexpr float kLog2eHost = 1.4426950408889634f;

// err: the library's device error word (see common.hpp), in every launcher.
hipError_t launch_quantize_append(const void* k, const void* v, int dtype, int n_new, int B, int H,
                                  int D, int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                  const float* signs, float rot_norm, int rot_kind, const float* lam,
                                  const float* vsigns, const int32_t* pos, unsigned* err,
                                  hipStream_t stream);

// Split pass arguments shared by both variants.
struct SplitArgs {
    const void* q;
    int dtype;
    int B, Hq, H, D, cap;
    uint8_t* kc;  // written only by the fused one-token append
    float* ks;
    uint8_t* vc;
    float* vs;
    const float* signs;
    float rot_norm;
    int rot_kind;      // with signs: 0 the Walsh-Hadamard rotation, 1 the FFT one
    const float* lam;  // K's per-channel scale [D] (q is divided by it), or null
    const int32_t* lens;
    int max_len;
    float qscale;  // softmax scale * log2(e): scores are kept in the log2 domain
    // Split s takes the pieces s, s + S, s + 2 S, ... of `chunk` tokens each
    // (one piece when S chunk >= max_len).  Tile it (32 tokens) of split s
    // starts at token s chunk + (it >> piece_shift) piece_stride +
    // (it & (2^piece_shift - 1)) 32, with piece_stride = S chunk and
    // 2^piece_shift = chunk / 32 tiles per piece; piece_shift = 30 when every
    // split has a single piece.
    int chunk;
    int num_splits;
    int piece_shift;
    int piece_stride;
    float* part_o;   // [B][Hq][S][D]
    float2* part_ml; // [B][Hq][S] (m, l)
    // block k = x + S (y + groups z) takes item items[k] = (split, sequence)
    // with KV-head group k % groups (longest first, written by the order
    // kernel), or null: block (x, y, z) takes split x of group y of sequence z
    const int2* items;
    // 1 when the token at lens[b] - 1 is appended by the combine of the same
    // call (the split pass then covers [0, lens[b] - 1)), else 0.
    int lens_offset;
    unsigned* err;  // the device error word
};

// 2- and 3-bit codes (plain bit-stream K rows, V in 32-token tiles): the append and the
// split pass; the combine is shared.
// The options of a b-bit append: K's rotation signs and kind, its channel
// scale, V's rotation signs (each null when off).
struct BitsRot {
    const float* signs;
    float rot_norm;
    int rot_kind;
    const float* lam;
    const float* vsigns;
};
hipError_t launch_quantize_bits(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                int cap, int bits, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                const int32_t* pos, const BitsRot& rot, unsigned* err, hipStream_t stream);
hipError_t launch_split_bits(const SplitArgs& a, int bits, hipStream_t stream);
// 2- and 3-bit codes on the matrix cores (head_dim 64, 128, 256; G <= 16; a
// rotated or channel-scaled K up to head_dim 128), and int4 codes at head_dim
// 192 (K plain or channel-scaled).
bool split_bits_mfma_supports(int D, int G, int bits, bool rotated_k, bool scaled_k);
int split_bits_mfma_heads_per_wave(int D, int G, int H, bool hilo);
hipError_t launch_split_bits_mfma(const SplitArgs& a, int bits, hipStream_t stream);

// Head widths that are multiples of 64 but not powers of two (192): the
// append (K optionally rotated by the mixed-radix FFT, V optionally too) and
// the split pass (any G <= 16) for the int4 layouts.
bool wide_supported_dim(int D);
// The bulk append kernel at head_dim 192 (8 or more tokens; K plain,
// channel-scaled or FFT-rotated, V not rotated).
bool quantize_tile_wide_supports(int D, int n_new, bool v_rotated);
hipError_t launch_quantize_tile_wide(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                     int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                     const float* signs, float rot_norm, const float* lam, const int32_t* pos,
                                     unsigned* err, hipStream_t stream);
hipError_t launch_quantize_wide(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs, const float* signs,
                                float rot_norm, const float* lam, const float* vsigns, const int32_t* pos,
                                unsigned* err, hipStream_t stream);
hipError_t launch_split_wide(const SplitArgs& a, hipStream_t stream);
// Returns hipErrorInvalidValue for (D, G) pairs the variant does not build.
hipError_t launch_split_vector(const SplitArgs& a, hipStream_t stream);
// Largest batch whose split blocks are ordered longest first.
constexpr int kOrderMaxBatch = 256;
// Writes items[S * groups * B] for batches of 2..kOrderMaxBatch sequences
// (see SplitArgs::items).
hipError_t launch_split_order(const int32_t* lens, int lens_offset, int max_len, int chunk, int S,
                              int groups, int B, int2* items, unsigned* err, hipStream_t stream);
hipError_t launch_split_mfma(const SplitArgs& a, hipStream_t stream);
bool split_vector_supports(int D, int G);
bool split_mfma_supports(int D, int G);
// KV heads one MFMA-variant workgroup serves (its grid has H / that blocks in y).
int split_mfma_heads_per_wave(int D, int G, int H);
// Waves per workgroup of the MFMA split kernel.
int split_mfma_block_waves(int D);

// Combine pass arguments.  With k_new set, the split pass covered
// [0, lens[b] - 1) and the combine quantises the token at lens[b] - 1 into
// the cache and merges it.
struct CombineArgs {
    const float* part_o;
    const float2* part_ml;
    const int32_t* lens;
    int max_len, chunk, S, B, Hq, D;
    float* out;
    // fused one-token append (k_new == nullptr: none)
    const uint16_t* k_new;  // [B][H][D]
    const uint16_t* v_new;
    const void* q;          // [B][Hq][D]
    int dtype, H, cap;
    uint8_t* kc;
    float* ks;
    uint8_t* vc;
    float* vs;
    const float* signs;
    float rot_norm;
    int rot_kind;           // with signs: 0 the Walsh-Hadamard rotation, 1 the FFT one
    const float* lam;       // K's per-channel scale [D], or null
    const float* vsigns;    // V's rotation signs [D] (same rot_norm), or null: the
                            // output is brought back to the original basis
    float qscale;           // softmax scale * log2(e)
    unsigned* err;          // the device error word
    int bits;               // code width of the appended token: 4, or 2 / 3
};
hipError_t launch_lse_combine(const CombineArgs& a, hipStream_t stream);

// The streaming-read probe: reads bytes / 16 uint4 of buf, writes blocks words.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);


}  // namespace otq
