// fp4q.hip -- gfx950 kernels and the C ABI of the FP4 communication-compression
// library (declared in include/fp4q.h).
//
// Method: "FP4Quant: Efficient 4-Bit Communication Compression for Model-Parallel
// LLM Training" (abstract): a hybrid two-level fast Walsh-Hadamard transform,
// micro-grouped dual-scale FP4 quantisation and cooperative FP4 packing on the
// sender; dequantisation, the inverse transform and (zot.news digest, "Read it
// as": the AllReduce of tensor parallelism) the sum of k peers on the receiver,
// or that sum (plus the rank's own uncompressed slice) quantised again for the
// all-gather half of the AllReduce.  A microscaling variant (32-element groups,
// power-of-two scales) sits beside the dual scale.
//
// Work mapping: one wavefront (64 lanes) handles a tile of 16 blocks of 256
// elements; lane l works on block p = l & 15 of the tile, together with the
// lanes l ^ 16, l ^ 32, l ^ 48 ("quarters" q = l >> 4).  Each lane keeps 64
// elements of its block in registers: six of the eight index bits of the block
// are register-index bits, the other two are lane bits 4 and 5 (= q).
//
// Transform: radix-2 stages in the order stride 1, 2, ..., 128 (index bit 0 to
// 7).  A stage on a register bit is a butterfly between two registers.  An index
// bit that sits in a lane bit is first brought into the registers, in exchange
// for an already transformed register bit, and then transformed in registers.
// The fp32-output receivers exchange with v_permlane16_swap (lane bit 4) or
// v_permlane32_swap (lane bit 5), one instruction per register pair; compress,
// whose time is VALU issue (a lane swap costs the issue slots of two adds), and
// the bf16-output receivers make their exchange through LDS instead.  The
// order of the exchanges is chosen per kernel so that
//   * decompress's payload loads of the four quarters cover whole 64-byte
//     segments per instruction (non-temporal path),
//   * compress ends with four whole micro-groups per lane, so group maxima,
//     scales, quantisation and packing stay in registers,
//   * the receiver ends with 16-byte register quads of contiguous output.
// Otherwise LDS only re-deals data between that lane-local layout and fully
// coalesced 1 KiB-per-instruction global accesses (the bf16 input tile, the
// peers' codes of the re-quantisation with a local slice, the codes and the
// output), in a region private to each wavefront.  No MFMA: the work is streaming and the transform
// is butterflies.
//
// The k-peer kernels whose time is their per-peer arithmetic use a narrow
// layout instead (8 blocks per wavefront, 32 elements per lane: each peer's
// codes in one contiguous 1 KiB load, half the registers, twice the resident
// wavefronts): the receiver reduce, and the re-quantisation without a local
// slice, which needs no transform at all.
//
// Numerics follow the method's fp32 operation order exactly (built with
// -ffp-contract=off, IEEE division, fp32 denormals kept):
//   * the transform runs on unscaled values z = 16 y; the 1/16 is folded into
//     the block maximum and the reciprocal scale, which is exact for bfloat16
//     inputs (every intermediate is a multiple of 2^-133, so scaling by 2^-4
//     never rounds, and z * (r / 16) is the same real number as (z / 16) * r);
//   * divisions use a hardware reciprocal estimate refined by fused
//     multiply-adds to the correctly rounded result; blocks whose largest
//     transformed value is below 2^-80 (where a remainder could underflow) take
//     the IEEE division instead;
//   * E4M3 micro-scales use the hardware RNE conversion after clamping to 448
//     (the conversion itself turns values above 464 into NaN);
//   * E2M1 codes use the hardware RNE conversion with scale 1 (its scale operand
//     only applies a power of two), which saturates at 6 and keeps the sign.
#include <hip/hip_runtime.h>

#include <float.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fp4q.h"
#include "fp4q_numerics.h"

namespace {

constexpr int kWave = 64;
constexpr int kTileBlocks = 16;  // 256-blocks per wavefront
// Wavefronts per workgroup (all LDS use is per wavefront).  The compute-heavy
// sender runs best with one wavefront per workgroup (more resident waves per
// CU); the store-heavy receivers with four (neighbouring tiles write
// neighbouring output from one CU), except decompress with bf16 output, which
// is compute-heavy too (kDecompressWaves).
#ifndef FP4Q_SENDER_WAVES
#define FP4Q_SENDER_WAVES 1
#endif
#ifndef FP4Q_RECEIVER_WAVES
#define FP4Q_RECEIVER_WAVES 4
#endif
#ifndef FP4Q_RECEIVER_ROUND
#define FP4Q_RECEIVER_ROUND 8
#endif
constexpr int kSenderWaves = FP4Q_SENDER_WAVES;
constexpr int kReceiverWaves = FP4Q_RECEIVER_WAVES;
// fp32 receiver output is staged kRoundBlocks blocks (65 chunks each) at a time
constexpr int kRoundBlocks = FP4Q_RECEIVER_ROUND;
// Decompress with bf16 output is bound by VALU issue more than by its stores, and
// like compress it runs faster with one wavefront per workgroup (more resident
// wavefronts per CU under the same LDS budget): 66.6 against 72.2 us at
// 32768 x 4096 (medians of three same-box runs).
#ifndef FP4Q_BF16_WAVES
#define FP4Q_BF16_WAVES 1
#endif
template <bool kBf16>
constexpr int kDecompressWaves = kBf16 ? FP4Q_BF16_WAVES : kReceiverWaves;


struct Lane {
    int lane;     // 0..63
    int p;        // block within the tile (lane bits 0-3)
    int q;        // quarter of the block held by this lane (lane bits 4-5)
    int64_t tile; // first block of the wavefront's tile (wave-uniform)
    int64_t b;    // flat block index
    int64_t bl;   // block to load: b, clamped to the last block for idle lanes
    bool valid;   // b < nblocks: only valid lanes store
};

// Lanes past the last block (a ragged final tile) load the last block instead
// and compute on it without storing, so no branch or zero fill is needed before
// the cross-lane exchanges (which need every lane).  nblocks >= 1.
template <int kWaves>
__device__ __forceinline__ Lane lane_map(int64_t nblocks) {
    Lane L;
    L.lane = threadIdx.x & (kWave - 1);
    const int wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    L.tile = ((int64_t)blockIdx.x * kWaves + wave_in_wg) * kTileBlocks;
    L.p = L.lane & 15;
    L.q = L.lane >> 4;
    L.b = L.tile + L.p;
    L.valid = L.b < nblocks;
    L.bl = L.valid ? L.b : nblocks - 1;
    return L;
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (byte selectors of
// the conversion builtins must be compile-time constants).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load on the non-temporal path (no allocation in the last-level cache).
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
// Global stores.  Every kernel writes through buffer stores, by default with
// the system-scope cache policy (sc1): on MI355X they wrote streaming output
// about 20 % faster than non-temporal global stores (6.1 against 4.9 TB/s on
// the decompress traffic pattern, 6.95 against 6.5 on the compress pattern).
// The k-peer reduce, whose eight read streams share the memory system with its
// one write stream, writes faster with the non-temporal policy instead.  A
// wavefront's descriptor covers exactly its tile's part of one output array:
// the bytes of its valid blocks, none for a wavefront whose tile lies past the
// last block (the last workgroup of a launch can hold such wavefronts), so a
// store past the end would also be dropped by the hardware range check; the
// kernels issue none.
constexpr int kStoreSc1 = 16;
constexpr int kStoreNt = 2;
template <int kPolicy>
struct TileStoreP {
    __amdgpu_buffer_rsrc_t r;
    // bytes_per_block of the array, for the tile's blocks [tile, tile + tile_blocks) that exist
    __device__ __forceinline__ TileStoreP(void *base, int64_t tile, int64_t nblocks,
                                          int bytes_per_block, int tile_blocks = kTileBlocks) {
        const int64_t left = nblocks - tile;
        const int64_t nvalid = left < 0 ? 0 : left < tile_blocks ? left : tile_blocks;
        r = __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(base) + tile * bytes_per_block, 0,
                                              static_cast<int>(nvalid * bytes_per_block), 0x00020000);
    }
    __device__ __forceinline__ void b128(int byte_offset, uint4 v) const {
        const u32x4 t = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(t, r, byte_offset, 0, kPolicy);
    }
    __device__ __forceinline__ void b32(int byte_offset, unsigned v) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_offset, 0, kPolicy);
    }
    __device__ __forceinline__ void b16(int byte_offset, unsigned short v) const {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, byte_offset, 0, kPolicy);
    }
    __device__ __forceinline__ void b8(int byte_offset, unsigned char v) const {
        __builtin_amdgcn_raw_buffer_store_b8(v, r, byte_offset, 0, kPolicy);
    }
};
#ifndef FP4Q_REDUCE_STORE_POLICY
#define FP4Q_REDUCE_STORE_POLICY kStoreNt
#endif
using TileStore = TileStoreP<kStoreSc1>;                     // scales: a few bytes per lane
using ReduceStore = TileStoreP<FP4Q_REDUCE_STORE_POLICY>;    // the k-peer reduce's output
// Codes and outputs (1 KiB per instruction): the transform kernels of the hot
// path write them with sc1 and the non-temporal policy together, the other
// kernels with sc1 alone (each the faster in its own steady state; a single
// launch on an idle GPU reads faster with sc1 alone, whose writes the
// last-level cache absorbs and drains after the kernel has ended).
// A build for a pipeline that runs other work between the kernels can give the
// transform kernels sc1 alone (-DFP4Q_HOT_STREAM_POLICY=16).
#ifndef FP4Q_HOT_STREAM_POLICY
#define FP4Q_HOT_STREAM_POLICY (kStoreSc1 | kStoreNt)
#endif
template <bool kHotTransform>
constexpr int kStreamPolicy = kHotTransform ? FP4Q_HOT_STREAM_POLICY : kStoreSc1;

// A buffer descriptor over the wavefront's tile of an array with
// bytes_per_block bytes per block: the bytes of the tile's nvalid existing
// blocks (built in scalar registers; loads outside it read zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, int64_t tile, int nvalid,
                                                            int bytes_per_block) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(reinterpret_cast<const char *>(base)) + tile * bytes_per_block, 0,
        nvalid * bytes_per_block, 0x00020000);
}
constexpr int kLoadNt = 2;  // the non-temporal cache policy

__device__ __forceinline__ float as_f(unsigned u) { return __uint_as_float(u); }
__device__ __forceinline__ unsigned as_u(float f) { return __float_as_uint(f); }

// Exchange lane bit 4 (odd/even 16-lane rows) with the register pair (a, b):
// afterwards a holds, in row parity L, what lane parity 0 held in register L,
// and b what lane parity 1 held in register L.
__device__ __forceinline__ void swap16(unsigned &a, unsigned &b) {
    auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// The same for lane bit 5 (upper / lower 32 lanes).
__device__ __forceinline__ void swap32(unsigned &a, unsigned &b) {
    auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(float &a, float &b) {
    unsigned x = as_u(a), y = as_u(b);
    swap16(x, y);
    a = as_f(x);
    b = as_f(y);
}
__device__ __forceinline__ void swap32(float &a, float &b) {
    unsigned x = as_u(a), y = as_u(b);
    swap32(x, y);
    a = as_f(x);
    b = as_f(y);
}

// One radix-2 stage between registers j and j + H.
template <int H>
__device__ __forceinline__ void stage(float (&R)[64]) {
#pragma unroll
    for (int j = 0; j < 64; ++j)
        if ((j & H) == 0) {
            const float a = R[j], b = R[j + H];
            R[j] = a + b;
            R[j + H] = a - b;
        }
}

// Exchange lane bit 4 (resp. 5) with register-index bit H, for all 32 pairs.
template <int H>
__device__ __forceinline__ void swap_lane4(float (&R)[64]) {
#pragma unroll
    for (int j = 0; j < 64; ++j)
        if ((j & H) == 0) swap16(R[j], R[j | H]);
}
template <int H>
__device__ __forceinline__ void swap_lane5(float (&R)[64]) {
#pragma unroll
    for (int j = 0; j < 64; ++j)
        if ((j & H) == 0) swap32(R[j], R[j | H]);
}

using fp4q_num::coarse_scale;
using fp4q_num::div_rn;
using fp4q_num::e2m1_pair;
using fp4q_num::e2m1_values;
using fp4q_num::e4m3_pair;
using fp4q_num::e4m3_value;
using fp4q_num::kE4M3Max;
using fp4q_num::rcp_rn;

// Maximum of v over the four lanes of a block (lane bits 4 and 5).
__device__ __forceinline__ float block_lane_max(float v) {
    float a = v, b = v;
    swap16(a, b);
    v = fmaxf(a, b);
    a = v;
    b = v;
    swap32(a, b);
    return fmaxf(a, b);
}

using fp4q_num::bf16_rne_pair;

// Wave-private LDS staging: a wavefront exchanges data among its own lanes
// through a region of 16-byte chunks (no workgroup barrier is needed; the
// fences keep the compiler from reordering LDS accesses across the exchange).
// Blocks are laid out with one chunk of padding (stride 33 chunks for 32 data
// chunks, 65 for 64, 9 for 8), so that both the scattered and the contiguous
// access patterns are free of bank conflicts and every address is a per-lane
// base plus a constant.
constexpr int kStageChunks = 528;  // 16 x 33 chunks = 8.25 KiB per wavefront
// receiver output staging: bf16 all 16 blocks of 33 chunks at once, fp32 in
// rounds of kRoundBlocks blocks of 65 chunks
template <bool kBf16>
constexpr int kReceiverChunks = kBf16 ? 16 * 33 : 65 * kRoundBlocks;

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- compress
// Input staging: the wavefront's tile (16 blocks of bf16, 8 KiB, contiguous)
// is read with eight fully coalesced 1 KiB loads into the wave-private LDS
// region, then each lane reads 128 bytes of its block.  The layout compress
// quantises from is register 16 k + i = element 16 q + 64 k + i: quarter q owns
// micro-groups q, q + 4, q + 8, q + 12 (index bits 0-3 and 6-7 in the register
// index, bits 4-5 in lane bits 4-5).  Without the transform the lane reads that
// layout straight from LDS.  With it, the first six stages need index bits 0-5
// in registers: the lane reads register j = element 64 q + j, transforms, and
// trades index bits 4-5 for 6-7 through LDS before the last two stages (the
// LDS pipe is idle there, while lane swaps would cost VALU issue slots, which
// bound this kernel).

// Two index bits held in lane bits 4-5 (call their value B) change places with
// the two index bits held in register bits kMoved, kMoved + 1 (value A), through
// the wavefront's LDS region (at least 528 chunks), in two rounds by register
// bit kRound, which stays put like register bits 0-2: round r writes the lane's
// 32 registers whose bit kRound is r as eight 16-byte chunks and reads eight
// back.  The chunk holding register bit 2 = c, A = a, B = b of block p sits at
// chunk 33 p + c + 2 a + 8 b: written by lane (p, q = b) from its registers with
// A = a, read by lane (p, q = a) into its registers with A = b.  The caller has
// finished any earlier use of the region.
template <int kMoved, int kRound>
__device__ __forceinline__ void exchange_through_lds(const Lane &L, uint4 *__restrict__ lds,
                                                     float (&R)[64]) {
    static_assert(kMoved >= 3 && kMoved + 1 <= 5 && kRound >= 3 && kRound <= 5 &&
                      kRound != kMoved && kRound != kMoved + 1,
                  "register bits 0-2 stay; kMoved, kMoved + 1 and kRound are the other three");
    uint4 *wr = lds + 33 * L.p + 8 * L.q;
    const uint4 *rd = lds + 33 * L.p + 2 * L.q;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        wave_lds_sync();
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = (a << kMoved) | (r << kRound) | (c << 2);
                wr[c + 2 * a] = make_uint4(as_u(R[j]), as_u(R[j + 1]), as_u(R[j + 2]), as_u(R[j + 3]));
            }
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint4 x = rd[c + 8 * b];
                const int j = (b << kMoved) | (r << kRound) | (c << 2);
                R[j] = as_f(x.x);
                R[j + 1] = as_f(x.y);
                R[j + 2] = as_f(x.z);
                R[j + 3] = as_f(x.w);
            }
    }
}

// The transform from the input layout (register j = element 64 q + j) to the
// quantisation layout; without the transform the input already has that layout.
template <bool kFwht>
__device__ __forceinline__ void compress_transform(const Lane &L, uint4 *__restrict__ lds,
                                                   float (&R)[64]) {
    if constexpr (kFwht) {
        stage<1>(R);   // level 1: index bits 0-3
        stage<2>(R);
        stage<4>(R);
        stage<8>(R);
        stage<16>(R);  // level 2: index bits 4-7
        stage<32>(R);
        // index bits 6-7 (lanes) for 4-5 (register bits 4-5): afterwards register
        // 16 k + i = element 16 q + 64 k + i
        exchange_through_lds<4, 3>(L, lds, R);
        stage<16>(R);  // index bit 6, now register bit 4
        stage<32>(R);  // index bit 7, now register bit 5
    }
}

// Scales and codes of the four register groups of a lane (registers
// 16 k .. 16 k + 15 form micro-group k; the four lanes of a block hold its 16
// groups).  kScaled: the registers hold 16 y (the transform's 1/16 not yet
// applied), which is folded into the block maximum and the reciprocals.
//   s  = max|y| / 2688 over the block;  t_k = max|y|_k / (6 s), clamped to 448;
//   mw = the four E4M3 micro-scales (byte k);  C = eight dwords of packed codes
//        (dword w covers registers 8 w .. 8 w + 7, low nibble first).
// The dual scales of a block from its largest |y|, A (already reduced over the
// block's lanes), and the lane's K group maxima a[k] (K even):
//   s = A / 2688;  t_k = a_k / (6 s), clamped to 448;  mw = the K E4M3
//   micro-scales (byte k);  inv[k] = 1 / (s * E4M3(m_k)), 0 for a zero scale.
template <int K>
__device__ __forceinline__ void dual_scales(float A, const float (&a)[K], float &s, float (&t)[K],
                                            unsigned &mw, float (&inv)[K]) {
    static_assert(K == 2 || K == 4, "two or four micro-groups per lane");
    const auto pack = [&]() {
        mw = e4m3_pair<false>(0u, t[0], t[1]);
        if constexpr (K == 4) mw = e4m3_pair<true>(mw, t[2], t[3]);
    };
    if (A >= 0x1p-80f) {
        s = coarse_scale(A);
        const float d6 = 6.0f * s;
        const float y = rcp_rn(d6);
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = fminf(div_rn(a[k], d6, y), kE4M3Max);
        pack();
        static_for<K>([&](auto k) {
            const float S = s * e4m3_value<decltype(k)::value>(mw);
            inv[k] = (S == 0.0f) ? 0.0f : rcp_rn(S);
        });
    } else {  // tiny or zero block: IEEE division throughout
        s = A / fp4q_num::kScaleDivisor;
        const float d6 = 6.0f * s;
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = (s != 0.0f) ? fminf(a[k] / d6, kE4M3Max) : 0.0f;
        pack();
        static_for<K>([&](auto k) {
            const float S = s * e4m3_value<decltype(k)::value>(mw);
            inv[k] = fminf((S == 0.0f) ? 0.0f : 1.0f / S, FLT_MAX);
        });
    }
}

// E2M1 codes of the lane's N registers, 16 per micro-group k (scale inv[k]):
// dword w of C covers registers 8 w .. 8 w + 7, low nibble first.
template <int N>
__device__ __forceinline__ void quantize_codes(const float (&R)[N], const float (&inv)[N / 16],
                                               unsigned (&C)[N / 8]) {
#pragma unroll
    for (int w = 0; w < N / 8; ++w) {
        const float r = inv[w >> 1];
        // the four conversions write all four bytes of c; starting from a
        // register that dies here (instead of 0) saves a move per dword
        unsigned c = as_u(R[8 * w]);
        static_for<4>([&](auto sel) {
            const int j = 8 * w + 2 * decltype(sel)::value;
            c = e2m1_pair<decltype(sel)::value>(c, R[j] * r, R[j + 1] * r);
        });
        C[w] = c;
    }
}

template <bool kScaled>
__device__ __forceinline__ void quantize_groups(const float (&R)[64], float &s, float (&t)[4],
                                                unsigned &mw, unsigned (&C)[8]) {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(R[16 * k + i]));
        a[k] = kScaled ? m * 0.0625f : m;
    }
    const float A = block_lane_max(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])));
    float inv[4];
    dual_scales<4>(A, a, s, t, mw, inv);
    if constexpr (kScaled) {
#pragma unroll
        for (int k = 0; k < 4; ++k) inv[k] *= 0.0625f;  // exact: the folded 1/16
    }
    quantize_codes<64>(R, inv, C);
}

// Codes of a tile through LDS (8 chunks per block, stride 9); the tile's 2 KiB
// of codes then leave in two 1 KiB stores.  The caller has finished any earlier
// use of the LDS region.  The lane's eight code dwords are in the quantisation
// layout (dword w = registers 8 w .. 8 w + 7 = elements 16 q + 64 (w >> 1) +
// 8 (w & 1) ..): C[w] is dword 2 q + 8 (w >> 1) + (w & 1) of the block, so
// C[2 m], C[2 m + 1] is one 8-byte write (chunk (q >> 1) + 2 m, dwords 2 (q & 1),
// + 1).
template <int kPolicy = kStoreSc1>
__device__ __forceinline__ void store_codes(const Lane &L, int64_t nblocks, uint4 *__restrict__ lds,
                                            uint4 *__restrict__ codes, const unsigned (&C)[8]) {
    const int lane = L.lane;
    uint2 *dst = reinterpret_cast<uint2 *>(lds + 9 * L.p + (L.q >> 1)) + (L.q & 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) dst[4 * m] = make_uint2(C[2 * m], C[2 * m + 1]);
    wave_lds_sync();
    const uint4 *srcl = lds + 9 * (lane >> 3) + (lane & 7);
    const TileStoreP<kPolicy> out(codes, L.tile, nblocks, 128);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int b = 8 * u + (lane >> 3);  // block within the tile
        const uint4 v = srcl[72 * u];
        if (L.tile + b < nblocks) out.b128(16 * (8 * b + (lane & 7)), v);
    }
}

// Tile loads: instruction j reads chunk 64 j + lane of the tile = chunk
// lane & 31 of block 2 j + (lane >> 5).  In a ragged last tile, blocks past the
// end re-read the last block (never stored).
__device__ __forceinline__ void load_tile(const uint4 *__restrict__ in, int64_t tile,
                                          int64_t nblocks, int lane, uint4 (&d)[8]) {
    if (tile + kTileBlocks <= nblocks) {
        const uint4 *src = in + tile * 32 + lane;
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = load_nt(src + 64 * j);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int64_t blk = tile + 2 * j + (lane >> 5);
            blk = blk < nblocks ? blk : nblocks - 1;
            d[j] = load_nt(in + blk * 32 + (lane & 31));
        }
    }
}

// The wavefront's bf16 tile staged through its LDS region (kStageChunks
// chunks); each lane then reads 128 bytes of its block p and widens them
// (exactly):
//   kGroups = false: register j = element 64 q + j (the lane's 128 contiguous bytes);
//   kGroups = true:  register 16 k + i = element 16 q + 64 k + i (four runs of 32 bytes).
template <bool kGroups>
__device__ __forceinline__ void load_widen(const Lane &L, const uint4 *__restrict__ in,
                                           int64_t nblocks, uint4 *__restrict__ lds,
                                           float (&R)[64]) {
    {
        uint4 d[8];
        load_tile(in, L.tile, nblocks, L.lane, d);
        uint4 *dst = lds + 33 * (L.lane >> 5) + (L.lane & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[66 * j] = d[j];
    }
    wave_lds_sync();
    const uint4 *srcl = lds + 33 * L.p + (kGroups ? 2 : 8) * L.q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // registers 8 i .. 8 i + 7 come from chunk i, or (grouped) chunk
        // 2 q + 8 (i >> 1) + (i & 1) of the block
        const uint4 x = srcl[kGroups ? 8 * (i >> 1) + (i & 1) : i];
        const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            R[8 * i + 2 * k] = as_f(w[k] << 16);
            R[8 * i + 2 * k + 1] = as_f(w[k] & 0xFFFF0000u);
        }
    }
}

template <bool kFwht>
__global__ __launch_bounds__(kWave * kSenderWaves) void compress_kernel(
    const uint4 *__restrict__ in, int64_t nblocks, uint4 *__restrict__ codes,
    unsigned *__restrict__ micro, float *__restrict__ block) {
    __shared__ uint4 lds_all[kSenderWaves * kStageChunks];
    const Lane L = lane_map<kSenderWaves>(nblocks);
    uint4 *lds = lds_all + (threadIdx.x / kWave) * kStageChunks;

    float R[64];
    load_widen<!kFwht>(L, in, nblocks, lds, R);
    compress_transform<kFwht>(L, lds, R);

    float s, t[4];
    unsigned mw, C[8];
    quantize_groups<kFwht>(R, s, t, mw, C);

    wave_lds_sync();  // every lane has read its chunks from the region
    // micro-scales: byte k of the quarter-q lane's mw is group q + 4k; its bytes
    // go to their places in the block's 16 bytes after the code staging (chunk
    // 144 + p), and the lane reads back groups 4q .. 4q + 3 once store_codes
    // has synchronised the region
    unsigned char *mb = reinterpret_cast<unsigned char *>(lds + 144 + L.p) + L.q;
#pragma unroll
    for (int k = 0; k < 4; ++k) mb[4 * k] = (unsigned char)(mw >> (8 * k));
    store_codes<kStreamPolicy<kFwht>>(L, nblocks, lds, codes, C);
    mw = reinterpret_cast<const unsigned *>(lds + 144 + L.p)[L.q];
    if (L.valid) {
        TileStore(micro, L.tile, nblocks, 16).b32(16 * L.p + 4 * L.q, mw);
        if (L.q == 0) TileStore(block, L.tile, nblocks, 4).b32(4 * L.p, as_u(s));
    }
}

// --------------------------------------------------- receiver: one payload
// Code layout in the lane: chunks q and q + 4 of its block (16 bytes = 32 codes
// each).  Decompress loads them so, instruction h of quarter q reading chunk
// q + 4 h: the four quarters read 64 contiguous bytes per instruction.  The
// re-quantisation with a local slice instead reads each peer's 2 KiB of tile
// codes as two contiguous 1 KiB loads and re-deals them through LDS
// (redeal_group_codes), into its own layout; for decompress's single payload
// that LDS round trip measured 7 % slower, on its one load round's critical path.
// Register j = 32 h + 8 w + t holds element 32 q + 128 h + 8 w + t: register
// bits 0-4 = index bits 0-4, bit 5 = index bit 7; lane bits 4, 5 = index bits
// 5, 6.  Its micro-group is (j >> 4 & 1) + 2 q + 8 h, so register group j >> 4
// uses micro byte 2 q + (j >> 4 & 1) + 8 (j >> 5).
// One lane's part of a payload: 32 code bytes, two micro-scale pairs, the block scale.
// (The re-quantisation's grouped layout keeps the same fields: dwords 2 k,
// 2 k + 1 of c0, c1 hold micro-group q + 4 k, lo and hi its bytes q, q + 4 and
// q + 8, q + 12.)
struct PayloadRegs {
    uint4 c0, c1;
    unsigned lo, hi;  // micro-scale bytes (2q, 2q + 1) and (2q + 8, 2q + 9) in the low halves
    float s;
};

// The block's 16 micro-scale bytes arrive in one 16-byte load (the four lanes of
// a block read the same 16 bytes); each lane keeps its two byte pairs.
__device__ __forceinline__ PayloadRegs load_payload(const Lane &L, const uint4 *__restrict__ codes,
                                                    const uint4 *__restrict__ micro,
                                                    const float *__restrict__ block) {
    PayloadRegs P;
    const uint4 *src = codes + L.bl * 8 + L.q;
    P.c0 = load_nt(src);
    P.c1 = load_nt(src + 4);
    const uint4 m = micro[L.bl];
    const unsigned sh = 16u * (L.q & 1);
    P.lo = ((L.q >> 1) ? m.y : m.x) >> sh;
    P.hi = ((L.q >> 1) ? m.w : m.z) >> sh;
    P.s = block[L.bl];
    return P;
}

// A peer's payload for the re-quantisation with a local slice, which sums in
// compress's quantisation layout (register 16 k + i = element 16 q + 64 k + i,
// micro-group q + 4 k), through buffer descriptors over the wavefront's tile:
// codes in the contiguous order (tile chunk 64 j + lane, chunk lane & 7 of
// block 8 j + (lane >> 3); redeal_group_codes gives the lane its groups), the
// block's 16 micro-scale bytes in one load, of which the lane keeps bytes q and
// q + 4 (lo) and q + 8 and q + 12 (hi), and the block scale.  Lanes of blocks
// past the end read zeros and never store.
__device__ __forceinline__ PayloadRegs load_payload_tile(const Lane &L, int64_t nblocks,
                                                         const uint4 *__restrict__ codes,
                                                         const uint4 *__restrict__ micro,
                                                         const float *__restrict__ block) {
    const int64_t left = nblocks - L.tile;
    const int nvalid = left <= 0 ? 0 : left < kTileBlocks ? (int)left : kTileBlocks;
    const __amdgpu_buffer_rsrc_t rc = tile_rsrc(codes, L.tile, nvalid, 128), rm = tile_rsrc(micro, L.tile, nvalid, 16);
    PayloadRegs P;
    const u32x4 c0 = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * L.lane, 0, kLoadNt);
    const u32x4 c1 = __builtin_amdgcn_raw_buffer_load_b128(rc, 1024 + 16 * L.lane, 0, kLoadNt);
    P.c0 = make_uint4(c0[0], c0[1], c0[2], c0[3]);
    P.c1 = make_uint4(c1[0], c1[1], c1[2], c1[3]);
    const u32x4 m = __builtin_amdgcn_raw_buffer_load_b128(rm, 16 * L.p, 0, 0);
    // byte q of dwords x, y (then z, w) into bytes 0, 1 (perm: selectors 0-3 pick
    // the second operand's bytes, 4-7 the first's)
    const unsigned sel = (unsigned)L.q | ((unsigned)(L.q + 4) << 8);
    P.lo = __builtin_amdgcn_perm(m[1], m[0], sel);
    P.hi = __builtin_amdgcn_perm(m[3], m[2], sel);
    P.s = as_f(__builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(block, L.tile, nvalid, 4), 4 * L.p, 0, 0));
    return P;
}

// Contiguously loaded codes to the quantisation layout through the wavefront's
// LDS region (at least 144 chunks, free): tile chunk c goes to chunk
// 9 (c >> 3) + (c & 7) (a padding chunk per block), and lane (p, q) reads the
// 8 bytes of each of its groups q + 4 k, half q & 1 of chunk (q >> 1) + 2 k of
// block p: dwords 2 k, 2 k + 1 of c0, c1.
__device__ __forceinline__ void redeal_group_codes(const Lane &L, uint4 *__restrict__ lds, PayloadRegs &P) {
    wave_lds_sync();  // earlier reads of the region are done
    uint4 *w = lds + 9 * (L.lane >> 3) + (L.lane & 7);
    w[0] = P.c0;
    w[72] = P.c1;
    wave_lds_sync();
    const uint2 *r = reinterpret_cast<const uint2 *>(lds + 9 * L.p + (L.q >> 1)) + (L.q & 1);
    const uint2 g0 = r[0], g1 = r[4], g2 = r[8], g3 = r[12];
    P.c0 = make_uint4(g0.x, g0.y, g1.x, g1.y);
    P.c1 = make_uint4(g2.x, g2.y, g3.x, g3.y);
}

// Registers j = 0..63 get E2M1(code) * S_g (kSet), or the product is added to
// them as a rounded product and a rounded sum (kAdd, the order the
// re-quantisation defines).
enum DequantMode { kSet, kAdd };
template <DequantMode kMode>
__device__ __forceinline__ void dequant(const PayloadRegs &P, float (&R)[64], float dscale = 1.0f) {
    const unsigned C[8] = {P.c0.x, P.c0.y, P.c0.z, P.c0.w, P.c1.x, P.c1.y, P.c1.z, P.c1.w};
    const float S[4] = {P.s * e4m3_value<0>(P.lo), P.s * e4m3_value<1>(P.lo),
                        P.s * e4m3_value<0>(P.hi), P.s * e4m3_value<1>(P.hi)};
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const float Sg = S[w >> 1];
        static_for<4>([&](auto sel) {
            const auto f = e2m1_values<decltype(sel)::value>(C[w], dscale);
            const int j = 8 * w + 2 * decltype(sel)::value;
            if constexpr (kMode == kAdd) {
                const float p0 = f[0] * Sg, p1 = f[1] * Sg;  // built without contraction
                R[j] = R[j] + p0;
                R[j + 1] = R[j + 1] + p1;
            } else {
                R[j] = f[0] * Sg;
                R[j + 1] = f[1] * Sg;
            }
        });
    }
}

// Inverse transform (the same butterflies) and the output layout.  Index bits
// 5 and 6 arrive in lane bits 4 and 5; they are exchanged with register bits
// chosen so that the output's 16-byte stores cover whole 64-byte segments:
//   fp32 out: with index bits 2, 3 -> register j of quarter q holds element
//     (j & 3) + 4 q + 32 (j >> 2 & 1) + 64 (j >> 3 & 1) + 16 (j >> 4 & 1)
//     + 128 (j >> 5), by lane swaps one bit at a time;
//   bf16 out: with index bits 3, 4 -> register j holds (j & 7) + 8 q + 32 (j >> 3),
//     through LDS, both bits at once: the region is free until the output
//     staging, and the exchange takes 64 lane swaps (128 VALU issue slots) off
//     the VALU (the fp32 receiver's region is sized for its output rounds, and
//     its stores bound it).
// Without the transform only the exchanges are made.  lds: the wavefront's
// region (kReceiverChunks<kBf16> chunks), free on entry; in use on return.
template <bool kFwht, bool kBf16>
__device__ __forceinline__ void receiver_transform(const Lane &L, uint4 *__restrict__ lds,
                                                   float (&R)[64], bool scaled = false) {
    if constexpr (kFwht) {
        stage<1>(R);   // index bits 0-4
        stage<2>(R);
        stage<4>(R);
        stage<8>(R);
        stage<16>(R);
    }
    if constexpr (kBf16) {
        exchange_through_lds<3, 5>(L, lds, R);
        wave_lds_sync();  // the region's reads are done before the output staging
        if constexpr (kFwht) {
            stage<8>(R);   // index bit 5
            stage<16>(R);  // index bit 6
        }
    } else {
        swap_lane4<4>(R);
        if constexpr (kFwht) stage<4>(R);  // index bit 5
        swap_lane5<8>(R);
        if constexpr (kFwht) stage<8>(R);  // index bit 6
    }
    if constexpr (kFwht) {
        stage<32>(R);  // index bit 7
        if (!scaled) {  // wave-uniform
#pragma unroll
            for (int j = 0; j < 64; ++j) R[j] *= 0.0625f;
        }
    }
}

// The transform's 1/16 may be applied by the FP4 decode instead (its scale
// operand is a power of two), which saves the 64 multiplies at the end: every
// value and partial sum is then exactly 1/16 of what the unscaled order
// computes, as long as none of them is subnormal.  Nonzero partial sums are
// multiples of the smallest unit in the last place among the block's decoded
// values, which is at least s * 2^-34 for block scale s (E2M1 >= 0.5, E4M3 >=
// 2^-9, 24-bit significands); so s >= 2^-80 on every lane of the wavefront
// keeps them all above 2^-114 and the result bit-identical.  The vote is
// wave-uniform, so both paths stay free of divergence.
__device__ __forceinline__ bool fold_sixteenth(float block_scale) {
    return __builtin_amdgcn_ballot_w64(block_scale >= 0x1p-80f) == ~0ull;
}

// Output staging: every lane's values go through the wave-private LDS region so
// that each global store instruction writes 1 KiB of contiguous output (64
// lanes x 16 bytes), the pattern the memory system absorbs fastest; kPolicy is
// the stores' cache policy.
template <bool kBf16, int kPolicy = kStoreSc1>
__device__ __forceinline__ void store_out(const Lane &L, int64_t nblocks, uint4 *__restrict__ lds,
                                          void *__restrict__ out, const float (&R)[64]) {
    const int lane = L.lane, p = L.p;
    const int64_t tile = L.tile;
    if constexpr (kBf16) {
        // a block is 32 chunks of 8 bf16 (stride 33); register 8v + t is chunk q + 4v
        uint4 *dst = lds + 33 * p + L.q;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int j = 8 * v;
            dst[4 * v] = make_uint4(bf16_rne_pair(R[j], R[j + 1]), bf16_rne_pair(R[j + 2], R[j + 3]),
                                    bf16_rne_pair(R[j + 4], R[j + 5]),
                                    bf16_rne_pair(R[j + 6], R[j + 7]));
        }
        wave_lds_sync();
        const uint4 *src = lds + 33 * (lane >> 5) + (lane & 31);
        const TileStoreP<kPolicy> dst_g(out, tile, nblocks, 512);
#pragma unroll
        for (int u = 0; u < 8; ++u) {  // blocks 2u, 2u + 1 of the tile
            const int b = 2 * u + (lane >> 5);
            const uint4 v = src[66 * u];
            if (tile + b < nblocks) dst_g.b128(16 * (32 * b + (lane & 31)), v);
        }
    } else {
        // a block is 64 chunks of 4 fp32 (stride 65); register quad v holds chunk
        // q + 8 (v & 1) + 16 (v >> 1 & 1) + 4 (v >> 2 & 1) + 32 (v >> 3).
        // Rounds of kRoundBlocks blocks each.
        const TileStoreP<kPolicy> dst_g(out, tile, nblocks, 1024);
#pragma unroll
        for (int h = 0; h < kTileBlocks / kRoundBlocks; ++h) {
            if (p / kRoundBlocks == h) {
                uint4 *dst = lds + 65 * (p % kRoundBlocks) + L.q;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = 4 * v;
                    const int c = 8 * (v & 1) + 16 * ((v >> 1) & 1) + 4 * ((v >> 2) & 1) + 32 * (v >> 3);
                    dst[c] = make_uint4(as_u(R[j]), as_u(R[j + 1]), as_u(R[j + 2]), as_u(R[j + 3]));
                }
            }
            wave_lds_sync();
            const uint4 *src = lds + lane;
#pragma unroll
            for (int u = 0; u < kRoundBlocks; ++u) {
                const int b = kRoundBlocks * h + u;
                const uint4 v = src[65 * u];
                if (tile + b < nblocks) dst_g.b128(16 * (64 * b + lane), v);
            }
            wave_lds_sync();
        }
    }
}

template <bool kFwht, bool kBf16>
__global__ __launch_bounds__(kWave * kDecompressWaves<kBf16>) void decompress_kernel(
    const uint4 *__restrict__ codes, const uint4 *__restrict__ micro,
    const float *__restrict__ block, int64_t nblocks, void *__restrict__ out) {
    __shared__ uint4 lds[kDecompressWaves<kBf16> * kReceiverChunks<kBf16>];
    const Lane L = lane_map<kDecompressWaves<kBf16>>(nblocks);
    float R[64];
    uint4 *wl = lds + (threadIdx.x / kWave) * kReceiverChunks<kBf16>;
    const PayloadRegs P = load_payload(L, codes, micro, block);
    const bool fold = kFwht && fold_sixteenth(P.s);
    dequant<kSet>(P, R, fold ? 0.0625f : 1.0f);
    receiver_transform<kFwht, kBf16>(L, wl, R, fold);
    store_out<kBf16, kStreamPolicy<kFwht>>(L, nblocks, wl, out, R);
}

// --------------------------------------------------- receiver-side reduce
struct Peers {
    const uint4 *codes[FP4Q_MAX_PEERS];
    const uint4 *micro[FP4Q_MAX_PEERS];
    const float *block[FP4Q_MAX_PEERS];
};

// add(load(p), first) for p = 0 .. k - 1 in order (first: an integral constant,
// true for peer 0 only), with the next peer's loads in flight while a peer is
// added (k >= 1, wave-uniform).  Two payload slots taken in turn, each reloaded
// unconditionally inside the loop, let every load write straight into the
// registers it is added from (a rolled loop with one slot, or a conditional
// reload, would copy the slot every peer).  The scheduling barriers keep each
// load issued before the previous peer's arithmetic (left alone, the compiler
// sinks it below that).
using First = std::integral_constant<bool, true>;
using Later = std::integral_constant<bool, false>;
template <typename Load, typename Add>
__device__ __forceinline__ void for_each_peer(int k, Load &&load, Add &&add) {
    auto A = load(0), B = A;
    if (k > 1) B = load(1);
    __builtin_amdgcn_sched_barrier(0);
    add(A, First{});
    int p = 1;  // B holds peer p
    for (; p + 2 < k; p += 2) {
        A = load(p + 1);
        __builtin_amdgcn_sched_barrier(0);
        add(B, Later{});
        B = load(p + 2);
        __builtin_amdgcn_sched_barrier(0);
        add(A, Later{});
    }
    if (p < k) {  // peer p (in B), and peer p + 1 if there is one
        const bool two = p + 1 < k;
        A = B;
        if (two) A = load(p + 1);
        __builtin_amdgcn_sched_barrier(0);
        add(B, Later{});
        if (two) add(A, Later{});
    }
}


// R += the k payloads (rounded products added in peer order), k >= 0.  Codes
// are loaded contiguously and re-dealt through the wavefront's LDS region lds
// (free during the sum, at least 144 chunks).  k is wave-uniform, so every
// branch here is uniform.
__device__ __forceinline__ void sum_peers(const Lane &L, int64_t nblocks, const Peers &peers, int k,
                                          uint4 *__restrict__ lds, float (&R)[64]) {
    if (k == 0) return;
    for_each_peer(
        k, [&](int p) { return load_payload_tile(L, nblocks, peers.codes[p], peers.micro[p], peers.block[p]); },
        [&](PayloadRegs &P, auto) {
            redeal_group_codes(L, lds, P);
            dequant<kAdd>(P, R);
        });
}


// ------------------------------------------- receiver-side re-quantisation
// Reduce-scatter step of a compressed AllReduce: the k payloads of a slice are
// summed where they live, in the transform domain (rounded products added in
// peer order), and the sum is quantised again with the compress steps -- no
// inverse transform is needed, since decompressing, summing and compressing
// would apply the self-inverse H / 16 twice.  With the rank's own uncompressed
// part of the slice (this kernel), the accumulator starts at that part,
// transformed exactly as compress transforms its input (its loads, its
// transform with the lane exchange through LDS, then the 1/16, exact for
// bfloat16 inputs), so the sum lives in compress's quantisation layout and
// leaves through compress's epilogue; without a local slice it starts at +0
// (requantize_narrow_kernel below).
template <bool kFwht>
__global__ __launch_bounds__(kWave * kReceiverWaves) void requantize_kernel(
    Peers peers, int k, const uint4 *__restrict__ local, int64_t nblocks,
    uint4 *__restrict__ codes, unsigned *__restrict__ micro, float *__restrict__ block) {
    __shared__ uint4 lds_all[kReceiverWaves * kStageChunks];
    const Lane L = lane_map<kReceiverWaves>(nblocks);
    uint4 *lds = lds_all + (threadIdx.x / kWave) * kStageChunks;
    float R[64];
    load_widen<!kFwht>(L, local, nblocks, lds, R);
    compress_transform<kFwht>(L, lds, R);
    if constexpr (kFwht) {
#pragma unroll
        for (int j = 0; j < 64; ++j) R[j] *= 0.0625f;
    }
    wave_lds_sync();  // every lane has read its chunks from the region
    sum_peers(L, nblocks, peers, k, lds, R);

    float s, t[4];
    unsigned mw, C[8];
    quantize_groups<false>(R, s, t, mw, C);
    wave_lds_sync();  // every lane has read its re-dealt codes
    // micro-scales to their stored order through the region, as compress does
    unsigned char *mb = reinterpret_cast<unsigned char *>(lds + 144 + L.p) + L.q;
#pragma unroll
    for (int g = 0; g < 4; ++g) mb[4 * g] = (unsigned char)(mw >> (8 * g));
    store_codes(L, nblocks, lds, codes, C);
    mw = reinterpret_cast<const unsigned *>(lds + 144 + L.p)[L.q];
    if (L.valid) {
        TileStore(micro, L.tile, nblocks, 16).b32(16 * L.p + 4 * L.q, mw);
        if (L.q == 0) TileStore(block, L.tile, nblocks, 4).b32(4 * L.p, as_u(s));
    }
}

// Without a local slice the re-quantisation applies no transform, so nothing
// ties a block's elements to one lane's registers across the whole block.  This
// kernel uses a narrow layout instead: a wavefront handles kNarrowBlocks = 8
// blocks and lane l works on block p = l >> 3 and its eighth e = l & 7, the 32
// elements [32 e, 32 e + 32) (micro-groups 2 e and 2 e + 1).  Every peer's codes
// for the tile then arrive in one contiguous 1 KiB load (16 bytes per lane),
// the new codes leave the same way, and micro-scales move as one 2-byte pair
// per lane: no LDS, 32 accumulator registers instead of 64, twice the resident
// wavefronts.  The block maximum is reduced over the block's eight lanes.
constexpr int kNarrowBlocks = 8;

struct NarrowLane {
    int lane, p, e;
    int64_t tile, b;
    int nvalid;           // blocks of the tile that exist (wave-uniform, 0 .. 8)
    unsigned oc, om, ob;  // byte offsets in the tile of the lane's codes, micro-scale pair, block scale
    bool valid;
};

// kEighthHigh: the eighth in lane bits 3-5 (p = lane bits 0-2), where the
// receivers' transform exchanges it; otherwise in lane bits 0-2.
template <int kWaves, bool kEighthHigh = false>
__device__ __forceinline__ NarrowLane narrow_map(int64_t nblocks) {
    NarrowLane L;
    L.lane = threadIdx.x & (kWave - 1);
    const int wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    L.tile = ((int64_t)blockIdx.x * kWaves + wave_in_wg) * kNarrowBlocks;
    L.p = kEighthHigh ? (L.lane & 7) : (L.lane >> 3);
    L.e = kEighthHigh ? (L.lane >> 3) : (L.lane & 7);
    L.b = L.tile + L.p;
    L.valid = L.b < nblocks;
    const int64_t left = nblocks - L.tile;
    L.nvalid = left <= 0 ? 0 : left < kNarrowBlocks ? (int)left : kNarrowBlocks;
    const unsigned chunk = (unsigned)L.p * 8u + (unsigned)L.e;
    L.oc = 16u * chunk;
    L.om = 2u * chunk;
    L.ob = 4u * (unsigned)L.p;
    return L;
}

// Maximum of v over the eight lanes of a block (lane bits 0-2), by swizzles
// within groups of 32 lanes (xor 1, 2, 4).
__device__ __forceinline__ float octet_max(float v) {
    v = fmaxf(v, as_f(__builtin_amdgcn_ds_swizzle(as_u(v), 0x041F)));
    v = fmaxf(v, as_f(__builtin_amdgcn_ds_swizzle(as_u(v), 0x081F)));
    return fmaxf(v, as_f(__builtin_amdgcn_ds_swizzle(as_u(v), 0x101F)));
}

struct NarrowPayload {
    uint4 c;     // 32 codes: elements 32 e .. 32 e + 31
    unsigned m;  // micro-scale bytes 2 e, 2 e + 1 in the low half
    float s;
};

// One peer's payload for the lane, through buffer descriptors over the
// wavefront's tile (built in scalar registers from the peer's base pointers, so
// a load costs no vector address arithmetic); lanes of blocks past the end read
// zeros (outside the descriptors' range) and never store.
__device__ __forceinline__ NarrowPayload load_narrow(const NarrowLane &L, const uint4 *__restrict__ codes,
                                                     const uint4 *__restrict__ micro,
                                                     const float *__restrict__ block) {
    NarrowPayload P;
    const u32x4 c =
        __builtin_amdgcn_raw_buffer_load_b128(tile_rsrc(codes, L.tile, L.nvalid, 128), (int)L.oc, 0, kLoadNt);
    P.c = make_uint4(c[0], c[1], c[2], c[3]);
    P.m = __builtin_amdgcn_raw_buffer_load_b16(tile_rsrc(micro, L.tile, L.nvalid, 16), (int)L.om, 0, 0);
    P.s = as_f(__builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(block, L.tile, L.nvalid, 4), (int)L.ob, 0, 0));
    return P;
}

// R[j] = R[j] + E2M1(code j) * S_g: a rounded product, then a rounded sum (the
// order the re-quantisation defines); kFirst: R[j] = +0 + E2M1(code j) * S_g.
template <bool kFirst>
__device__ __forceinline__ void dequant_add_narrow(const NarrowPayload &P, float (&R)[32]) {
    const unsigned C[4] = {P.c.x, P.c.y, P.c.z, P.c.w};
    const float S[2] = {P.s * e4m3_value<0>(P.m), P.s * e4m3_value<1>(P.m)};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float Sg = S[w >> 1];
        static_for<4>([&](auto sel) {
            const auto f = e2m1_values<decltype(sel)::value>(C[w]);
            const int j = 8 * w + 2 * decltype(sel)::value;
            const float p0 = f[0] * Sg, p1 = f[1] * Sg;  // built without contraction
            R[j] = (kFirst ? 0.0f : R[j]) + p0;
            R[j + 1] = (kFirst ? 0.0f : R[j + 1]) + p1;
        });
        __builtin_amdgcn_sched_barrier(0);  // decode no further ahead than a dword
    }
}

__global__ __launch_bounds__(kWave * kReceiverWaves) void requantize_narrow_kernel(
    Peers peers, int k, int64_t nblocks, uint4 *__restrict__ codes, unsigned short *__restrict__ micro,
    float *__restrict__ block) {
    const NarrowLane L = narrow_map<kReceiverWaves>(nblocks);
    float R[32];
    for_each_peer(
        k, [&](int p) { return load_narrow(L, peers.codes[p], peers.micro[p], peers.block[p]); },
        [&](const NarrowPayload &P, auto first) { dequant_add_narrow<decltype(first)::value>(P, R); });

    float a[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(R[16 * g + i]));
        a[g] = m;
    }
    const float A = octet_max(fmaxf(a[0], a[1]));
    float s, t[2], inv[2];
    unsigned mw, C[4];
    dual_scales<2>(A, a, s, t, mw, inv);
    quantize_codes<32>(R, inv, C);
    if (L.valid) {
        TileStore(codes, L.tile, nblocks, 128, kNarrowBlocks).b128(16 * L.lane, make_uint4(C[0], C[1], C[2], C[3]));
        TileStore(micro, L.tile, nblocks, 16, kNarrowBlocks).b16(16 * L.p + 2 * L.e, (unsigned short)(mw & 0xFFFFu));
        if (L.e == 0) TileStore(block, L.tile, nblocks, 4, kNarrowBlocks).b32(4 * L.p, as_u(s));
    }
}

// ------------------------------------------- receiver reduce, narrow layout
// Eight blocks per wavefront; lane l works on block p = l & 7 and its eighth
// e = l >> 3 (element bits 5-7 in lane bits 3-5): 32 accumulator registers
// (element bits 0-4).  Every peer's codes arrive in one contiguous 1 KiB load.
// The inverse transform runs its first five stages in registers, then brings
// element bits 5, 6 and 7 into register bit 4 one at a time -- lane bit 3 by a
// row rotation (DPP), lane bits 4 and 5 by lane swaps -- each followed by its
// stage; afterwards register r holds element (r & 15) + 16 f + 128 (r >> 4),
// f = l >> 3, i.e. two runs of 16 consecutive values per lane.

// Exchange lane bit 3 with register bit 4 (pairs r, r + 16): lanes with bit 3
// clear receive the partner's r into r + 16, lanes with it set the partner's
// r + 16 into r (DPP row rotation by 8 = the lane eight apart, written per bank).
__device__ __forceinline__ void swap_lane3_reg4(float (&R)[32]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const unsigned a = as_u(R[r]), b = as_u(R[r + 16]);
        const unsigned b2 = (unsigned)__builtin_amdgcn_update_dpp((int)b, (int)a, 0x128, 0xF, 0x3, false);
        const unsigned a2 = (unsigned)__builtin_amdgcn_update_dpp((int)a, (int)b, 0x128, 0xF, 0xC, false);
        R[r] = as_f(a2);
        R[r + 16] = as_f(b2);
    }
}

template <int H>
__device__ __forceinline__ void stage32(float (&R)[32]) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
        if ((j & H) == 0) {
            const float a = R[j], b = R[j + H];
            R[j] = a + b;
            R[j + H] = a - b;
        }
}

template <bool kFwht>
__device__ __forceinline__ void narrow_receiver_transform(float (&R)[32]) {
    if constexpr (kFwht) {
        stage32<1>(R);
        stage32<2>(R);
        stage32<4>(R);
        stage32<8>(R);
        stage32<16>(R);   // element bit 4
    }
    swap_lane3_reg4(R);
    if constexpr (kFwht) stage32<16>(R);  // element bit 5
#pragma unroll
    for (int r = 0; r < 16; ++r) swap16(R[r], R[r + 16]);
    if constexpr (kFwht) stage32<16>(R);  // element bit 6
#pragma unroll
    for (int r = 0; r < 16; ++r) swap32(R[r], R[r + 16]);
    if constexpr (kFwht) {
        stage32<16>(R);  // element bit 7
#pragma unroll
        for (int j = 0; j < 32; ++j) R[j] *= 0.0625f;
    }
}

// R[j] = R[j] + E2M1(code j) * S_g with one fused multiply-add (kFirst: added
// to +0).
template <bool kFirst>
__device__ __forceinline__ void dequant_fma_narrow(const NarrowPayload &P, float (&R)[32]) {
    const unsigned C[4] = {P.c.x, P.c.y, P.c.z, P.c.w};
    const float S[2] = {P.s * e4m3_value<0>(P.m), P.s * e4m3_value<1>(P.m)};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float Sg = S[w >> 1];
        static_for<4>([&](auto sel) {
            const auto f = e2m1_values<decltype(sel)::value>(C[w]);
            const int j = 8 * w + 2 * decltype(sel)::value;
            R[j] = fmaf(f[0], Sg, kFirst ? 0.0f : R[j]);
            R[j + 1] = fmaf(f[1], Sg, kFirst ? 0.0f : R[j + 1]);
        });
        __builtin_amdgcn_sched_barrier(0);  // decode no further ahead than a dword
    }
}

constexpr int kNarrowOutChunks = 264;  // fp32: 4 blocks of 65 chunks; bf16: 8 of 33

// Output through the wavefront's LDS region so that every store writes 1 KiB.
template <bool kBf16>
__device__ __forceinline__ void narrow_store_out(const NarrowLane &L, int64_t nblocks, uint4 *__restrict__ lds,
                                                 void *__restrict__ out, const float (&R)[32]) {
    const int lane = L.lane, p = L.p, f = L.e;
    if constexpr (kBf16) {
        // a block is 32 chunks of 8 bf16 (stride 33); run h (registers 16 h ..) is
        // chunks 16 h + 2 f, + 1
        uint4 *dst = lds + 33 * p + 2 * f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = 16 * h + 8 * c;
                dst[16 * h + c] = make_uint4(bf16_rne_pair(R[j], R[j + 1]), bf16_rne_pair(R[j + 2], R[j + 3]),
                                             bf16_rne_pair(R[j + 4], R[j + 5]), bf16_rne_pair(R[j + 6], R[j + 7]));
            }
        wave_lds_sync();
        const uint4 *src = lds + 33 * (lane >> 5) + (lane & 31);
        const ReduceStore dst_g(out, L.tile, nblocks, 512, kNarrowBlocks);
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // blocks 2u, 2u + 1
            const int b = 2 * u + (lane >> 5);
            const uint4 v = src[66 * u];
            if (L.tile + b < nblocks) dst_g.b128(16 * (32 * b + (lane & 31)), v);
        }
    } else {
        // a block is 64 chunks of 4 fp32 (stride 65); run h is chunks 32 h + 4 f .. + 3;
        // two rounds of four blocks
        const ReduceStore dst_g(out, L.tile, nblocks, 1024, kNarrowBlocks);
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            if ((p >> 2) == rd) {
                uint4 *dst = lds + 65 * (p & 3) + 4 * f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int j = 16 * h + 4 * c;
                        dst[32 * h + c] = make_uint4(as_u(R[j]), as_u(R[j + 1]), as_u(R[j + 2]), as_u(R[j + 3]));
                    }
            }
            wave_lds_sync();
            const uint4 *src = lds + lane;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = 4 * rd + u;
                const uint4 v = src[65 * u];
                if (L.tile + b < nblocks) dst_g.b128(16 * (64 * b + lane), v);
            }
            wave_lds_sync();
        }
    }
}

template <bool kFwht, bool kBf16>
__global__ __launch_bounds__(kWave * kReceiverWaves) void accumulate_narrow_kernel(
    Peers peers, int k, int64_t nblocks, void *__restrict__ out) {
    __shared__ uint4 lds[kReceiverWaves * kNarrowOutChunks];
    const NarrowLane L = narrow_map<kReceiverWaves, true>(nblocks);
    uint4 *wl = lds + (threadIdx.x / kWave) * kNarrowOutChunks;
    float R[32];
    for_each_peer(
        k, [&](int p) { return load_narrow(L, peers.codes[p], peers.micro[p], peers.block[p]); },
        [&](const NarrowPayload &P, auto first) { dequant_fma_narrow<decltype(first)::value>(P, R); });
    narrow_receiver_transform<kFwht>(R);
    narrow_store_out<kBf16>(L, nblocks, wl, out, R);
}

// --------------------------------------------------- MXFP4-style variant
// Every 32 consecutive transformed values share one power-of-two scale 2^e,
// e = floor(log2 max|y|) - 2 clamped to [-127, 127] (-127 for a zero group),
// stored as an E8M0 byte e + 127; elements are E2M1(y / 2^e).  The conversion
// instruction divides by the power of two of its scale operand, so the scale
// costs no multiply.  After compress_transform a 32-group (index bits 0-4) is
// register group k (bits 0-3) of the two quarters q, q ^ 1 (lane bit 4 = bit 4);
// its number within the block is (q >> 1) + 2 k.
__device__ __forceinline__ float pair_lane_max(float v) {  // max over lane bit 4
    float a = v, b = v;
    swap16(a, b);
    return fmaxf(a, b);
}

template <bool kFwht>
__global__ __launch_bounds__(kWave * kSenderWaves) void compress_mx_kernel(
    const uint4 *__restrict__ in, int64_t nblocks, uint4 *__restrict__ codes,
    uint8_t *__restrict__ scales) {
    __shared__ uint4 lds_all[kSenderWaves * kStageChunks];
    const Lane L = lane_map<kSenderWaves>(nblocks);
    uint4 *lds = lds_all + (threadIdx.x / kWave) * kStageChunks;
    const int q = L.q;
    float R[64];
    load_widen<!kFwht>(L, in, nblocks, lds, R);
    compress_transform<kFwht>(L, lds, R);

    // exponent of each 32-group; the registers hold 16 y when transformed
    int e[4];
    float scale[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(R[16 * k + i]));
        m = pair_lane_max(m);
        // floor(log2 m) = exponent field - 127 for normal m; zero or subnormal m
        // clamps to -127 below.  16 y is exact, so floor(log2 max|y|) is 4 less.
        int ek = (int)(as_u(m) >> 23) - 127 - (kFwht ? 4 : 0) - 2;
        ek = ek < -127 ? -127 : (ek > 127 ? 127 : ek);
        e[k] = ek;
        // divisor applied by the conversion: 2^e (times 16 for 16 y), a normal
        // float except for e = -127 without the transform: then the group's
        // values (all below 2^-124) are doubled exactly and 2^-126 is used
        int sh = ek + (kFwht ? 4 : 0);
        if (!kFwht && sh == -127) {
#pragma unroll
            for (int i = 0; i < 16; ++i) R[16 * k + i] *= 2.0f;
            sh = -126;
        }
        scale[k] = as_f((unsigned)(sh + 127) << 23);
    }

    unsigned C[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const float sc = scale[w >> 1];
        unsigned c = as_u(R[8 * w]);  // every byte is written below (as in compress)
        static_for<4>([&](auto sel) {
            const int j = 8 * w + 2 * decltype(sel)::value;
            c = e2m1_pair<decltype(sel)::value>(c, R[j], R[j + 1], sc);
        });
        C[w] = c;
    }
    wave_lds_sync();  // every lane has read its chunks from the region
    store_codes(L, nblocks, lds, codes, C);
    if (L.valid && (q & 1) == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            TileStore(scales, L.tile, nblocks, 8).b8(8 * L.p + (q >> 1) + 2 * k, (unsigned char)(e[k] + 127));
    }
}

// Receiver: register j of quarter q holds element 32 q + 128 (j >> 5) + (j & 31),
// whose 32-group is q + 4 (j >> 5).
template <bool kFwht, bool kBf16>
__global__ __launch_bounds__(kWave * kReceiverWaves) void decompress_mx_kernel(
    const uint4 *__restrict__ codes, const uint2 *__restrict__ scales, int64_t nblocks,
    void *__restrict__ out) {
    __shared__ uint4 lds[kReceiverWaves * kReceiverChunks<kBf16>];
    const Lane L = lane_map<kReceiverWaves>(nblocks);
    const uint4 *src = codes + L.bl * 8 + L.q;
    const uint4 c0 = load_nt(src), c1 = load_nt(src + 4);
    const uint2 sw = scales[L.bl];  // the block's 8 scale bytes
    const int e0 = (int)((sw.x >> (8 * L.q)) & 0xFFu) - 127;  // group q
    const int e1 = (int)((sw.y >> (8 * L.q)) & 0xFFu) - 127;  // group q + 4
    const unsigned C[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    // the transform's 1/16 goes into the decode scale when every group's
    // exponent is at least -100: decoded values are multiples of 2^(e - 1), so
    // no value or partial sum comes near the subnormal range (see
    // fold_sixteenth); the vote is wave-uniform
    const bool fold = kFwht && __builtin_amdgcn_ballot_w64(e0 >= -100 && e1 >= -100) == ~0ull;
    float R[64];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = (h ? e1 : e0) - (fold ? 4 : 0);
        // 2^e as the conversion's scale; 2^-127 is subnormal, so use 2^-126 and halve
        const float sc = as_f((unsigned)((e < -126 ? -126 : e) + 127) << 23);
#pragma unroll
        for (int w = 4 * h; w < 4 * h + 4; ++w) {
            static_for<4>([&](auto sel) {
                const auto f = e2m1_values<decltype(sel)::value>(C[w], sc);
                const int j = 8 * w + 2 * decltype(sel)::value;
                R[j] = f[0];
                R[j + 1] = f[1];
            });
        }
        if (e < -126) {
#pragma unroll
            for (int j = 32 * h; j < 32 * h + 32; ++j) R[j] *= 0.5f;  // exact
        }
    }
    uint4 *wl = lds + (threadIdx.x / kWave) * kReceiverChunks<kBf16>;
    receiver_transform<kFwht, kBf16>(L, wl, R, fold);
    store_out<kBf16>(L, nblocks, wl, out, R);
}

// ------------------------------------------------------------------- host
inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;
};
inline Range rng(const void *p, int64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Validates the shape; on success sets n (elements) and nb (blocks).
int check_shape(int64_t rows, int64_t row_len, int64_t *n, int64_t *nb) {
    if (rows < 0 || row_len <= 0 || row_len % FP4Q_BLOCK != 0) return FP4Q_ERR_SHAPE;
    // fp32 output bytes = 4 * rows * row_len must fit in int64
    if (rows > 0 && row_len > INT64_MAX / 4 / rows) return FP4Q_ERR_SHAPE;
    *n = rows * row_len;
    *nb = *n / FP4Q_BLOCK;
    // grid: one workgroup per 64 blocks
    if ((*nb + kTileBlocks - 1) / kTileBlocks > (int64_t)0x7FFFFFFF) return FP4Q_ERR_SHAPE;
    return FP4Q_OK;
}

int launch(const void *fn, int64_t nb, int waves, void **args, void *stream,
           int tile_blocks = kTileBlocks) {
    const int64_t per_wg = (int64_t)tile_blocks * waves;
    const dim3 grid((unsigned)((nb + per_wg - 1) / per_wg)), threads(kWave * waves);
    const hipError_t e = hipLaunchKernel(fn, grid, threads, args, 0, (hipStream_t)stream);
    return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_LAUNCH;
}

int check_payload_ptrs(const void *codes, const void *micro, const void *block) {
    if (!codes || !micro || !block) return FP4Q_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(micro, 16) || !aligned(block, 4)) return FP4Q_ERR_ALIGN;
    return FP4Q_OK;
}

}  // namespace

extern "C" {

int fp4q_payload_bytes(int64_t rows, int64_t row_len, size_t *codes_bytes, size_t *micro_bytes,
                       size_t *block_bytes) {
    int64_t n, nb;
    const int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (codes_bytes) *codes_bytes = (size_t)(n / 2);
    if (micro_bytes) *micro_bytes = (size_t)(n / FP4Q_GROUP);
    if (block_bytes) *block_bytes = (size_t)(nb * 4);
    return FP4Q_OK;
}

int fp4q_compress_ex(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                     uint8_t *micro_scales, float *block_scales, uint32_t flags, void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if (!in_bf16) return FP4Q_ERR_NULL;
    if ((st = check_payload_ptrs(codes, micro_scales, block_scales)) != FP4Q_OK) return st;
    if (!aligned(in_bf16, 16)) return FP4Q_ERR_ALIGN;
    const Range in = rng(in_bf16, 2 * n), c = rng(codes, n / 2), m = rng(micro_scales, n / 16),
                b = rng(block_scales, 4 * nb);
    if (overlap(in, c) || overlap(in, m) || overlap(in, b) || overlap(c, m) || overlap(c, b) ||
        overlap(m, b))
        return FP4Q_ERR_ARG;
    void *args[] = {&in_bf16, &nb, &codes, &micro_scales, &block_scales};
    const void *fn = (flags & FP4Q_FLAG_NO_FWHT) ? (const void *)&compress_kernel<false>
                                                 : (const void *)&compress_kernel<true>;
    return launch(fn, nb, kSenderWaves, args, stream);
}

int fp4q_compress(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                  uint8_t *micro_scales, float *block_scales, void *stream) {
    return fp4q_compress_ex(in_bf16, rows, row_len, codes, micro_scales, block_scales, 0u, stream);
}

int fp4q_decompress_ex(const uint8_t *codes, const uint8_t *micro_scales,
                       const float *block_scales, int64_t rows, int64_t row_len, void *out,
                       int out_dtype, uint32_t flags, void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (out_dtype != FP4Q_OUT_F32 && out_dtype != FP4Q_OUT_BF16) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if ((st = check_payload_ptrs(codes, micro_scales, block_scales)) != FP4Q_OK) return st;
    if (!out) return FP4Q_ERR_NULL;
    if (!aligned(out, 16)) return FP4Q_ERR_ALIGN;
    const Range o = rng(out, (out_dtype == FP4Q_OUT_F32 ? 4 : 2) * n);
    if (overlap(o, rng(codes, n / 2)) || overlap(o, rng(micro_scales, n / 16)) ||
        overlap(o, rng(block_scales, 4 * nb)))
        return FP4Q_ERR_ARG;
    void *args[] = {&codes, &micro_scales, &block_scales, &nb, &out};
    const bool fw = !(flags & FP4Q_FLAG_NO_FWHT), bf = out_dtype == FP4Q_OUT_BF16;
    const void *fn = fw ? (bf ? (const void *)&decompress_kernel<true, true>
                              : (const void *)&decompress_kernel<true, false>)
                        : (bf ? (const void *)&decompress_kernel<false, true>
                              : (const void *)&decompress_kernel<false, false>);
    return launch(fn, nb, bf ? kDecompressWaves<true> : kReceiverWaves, args, stream);
}

int fp4q_decompress(const uint8_t *codes, const uint8_t *micro_scales, const float *block_scales,
                    int64_t rows, int64_t row_len, float *out_f32, void *stream) {
    return fp4q_decompress_ex(codes, micro_scales, block_scales, rows, row_len, out_f32,
                              FP4Q_OUT_F32, 0u, stream);
}

int fp4q_decompress_accumulate_ex(int k, const uint8_t *const *codes,
                                  const uint8_t *const *micro_scales,
                                  const float *const *block_scales, int64_t rows,
                                  int64_t row_len, void *out, int out_dtype, uint32_t flags,
                                  void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (k < 1 || k > FP4Q_MAX_PEERS) return FP4Q_ERR_K;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (out_dtype != FP4Q_OUT_F32 && out_dtype != FP4Q_OUT_BF16) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if (!codes || !micro_scales || !block_scales || !out) return FP4Q_ERR_NULL;
    if (!aligned(out, 16)) return FP4Q_ERR_ALIGN;
    const Range o = rng(out, (out_dtype == FP4Q_OUT_F32 ? 4 : 2) * n);
    Peers peers = {};
    for (int p = 0; p < k; ++p) {
        if ((st = check_payload_ptrs(codes[p], micro_scales[p], block_scales[p])) != FP4Q_OK)
            return st;
        if (overlap(o, rng(codes[p], n / 2)) || overlap(o, rng(micro_scales[p], n / 16)) ||
            overlap(o, rng(block_scales[p], 4 * nb)))
            return FP4Q_ERR_ARG;
        peers.codes[p] = reinterpret_cast<const uint4 *>(codes[p]);
        peers.micro[p] = reinterpret_cast<const uint4 *>(micro_scales[p]);
        peers.block[p] = block_scales[p];
    }
    void *args[] = {&peers, &k, &nb, &out};
    const bool fw = !(flags & FP4Q_FLAG_NO_FWHT), bf = out_dtype == FP4Q_OUT_BF16;
    const void *fn = fw ? (bf ? (const void *)&accumulate_narrow_kernel<true, true>
                              : (const void *)&accumulate_narrow_kernel<true, false>)
                        : (bf ? (const void *)&accumulate_narrow_kernel<false, true>
                              : (const void *)&accumulate_narrow_kernel<false, false>);
    return launch(fn, nb, kReceiverWaves, args, stream, kNarrowBlocks);
}

int fp4q_decompress_accumulate(int k, const uint8_t *const *codes,
                               const uint8_t *const *micro_scales,
                               const float *const *block_scales, int64_t rows, int64_t row_len,
                               void *out, int out_dtype, void *stream) {
    return fp4q_decompress_accumulate_ex(k, codes, micro_scales, block_scales, rows, row_len, out,
                                         out_dtype, 0u, stream);
}

int fp4q_reduce_requantize_ex(int k, const uint8_t *const *codes,
                              const uint8_t *const *micro_scales,
                              const float *const *block_scales, const uint16_t *local_bf16,
                              int64_t rows, int64_t row_len, uint8_t *out_codes,
                              uint8_t *out_micro, float *out_block, uint32_t flags,
                              void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (k < (local_bf16 ? 0 : 1) || k > FP4Q_MAX_PEERS) return FP4Q_ERR_K;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if (k > 0 && (!codes || !micro_scales || !block_scales)) return FP4Q_ERR_NULL;
    if ((st = check_payload_ptrs(out_codes, out_micro, out_block)) != FP4Q_OK) return st;
    if (local_bf16 && !aligned(local_bf16, 16)) return FP4Q_ERR_ALIGN;
    const Range oc = rng(out_codes, n / 2), om = rng(out_micro, n / 16), ob = rng(out_block, 4 * nb);
    if (overlap(oc, om) || overlap(oc, ob) || overlap(om, ob)) return FP4Q_ERR_ARG;
    if (local_bf16) {
        const Range il = rng(local_bf16, 2 * n);
        if (overlap(oc, il) || overlap(om, il) || overlap(ob, il)) return FP4Q_ERR_ARG;
    }
    Peers peers = {};
    for (int p = 0; p < k; ++p) {
        if ((st = check_payload_ptrs(codes[p], micro_scales[p], block_scales[p])) != FP4Q_OK)
            return st;
        const Range ic = rng(codes[p], n / 2), im = rng(micro_scales[p], n / 16),
                    ib = rng(block_scales[p], 4 * nb);
        for (const Range o : {oc, om, ob})
            if (overlap(o, ic) || overlap(o, im) || overlap(o, ib)) return FP4Q_ERR_ARG;
        peers.codes[p] = reinterpret_cast<const uint4 *>(codes[p]);
        peers.micro[p] = reinterpret_cast<const uint4 *>(micro_scales[p]);
        peers.block[p] = block_scales[p];
    }
    if (!local_bf16) {  // no transform anywhere: the narrow layout
        void *args[] = {&peers, &k, &nb, &out_codes, &out_micro, &out_block};
        return launch((const void *)&requantize_narrow_kernel, nb, kReceiverWaves, args, stream,
                      kNarrowBlocks);
    }
    void *args[] = {&peers, &k, &local_bf16, &nb, &out_codes, &out_micro, &out_block};
    const bool fw = !(flags & FP4Q_FLAG_NO_FWHT);
    const void *fn = fw ? (const void *)&requantize_kernel<true> : (const void *)&requantize_kernel<false>;
    return launch(fn, nb, kReceiverWaves, args, stream);
}

int fp4q_reduce_requantize(int k, const uint8_t *const *codes, const uint8_t *const *micro_scales,
                           const float *const *block_scales, int64_t rows, int64_t row_len,
                           uint8_t *out_codes, uint8_t *out_micro, float *out_block,
                           void *stream) {
    return fp4q_reduce_requantize_ex(k, codes, micro_scales, block_scales, nullptr, rows, row_len,
                                     out_codes, out_micro, out_block, 0u, stream);
}

int fp4q_compress_mx(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                     uint8_t *scales, uint32_t flags, void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if (!in_bf16 || !codes || !scales) return FP4Q_ERR_NULL;
    if (!aligned(in_bf16, 16) || !aligned(codes, 16) || !aligned(scales, 8)) return FP4Q_ERR_ALIGN;
    const Range in = rng(in_bf16, 2 * n), c = rng(codes, n / 2), sc = rng(scales, n / 32);
    if (overlap(in, c) || overlap(in, sc) || overlap(c, sc)) return FP4Q_ERR_ARG;
    void *args[] = {&in_bf16, &nb, &codes, &scales};
    const void *fn = (flags & FP4Q_FLAG_NO_FWHT) ? (const void *)&compress_mx_kernel<false>
                                                 : (const void *)&compress_mx_kernel<true>;
    return launch(fn, nb, kSenderWaves, args, stream);
}

int fp4q_decompress_mx(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t row_len,
                       void *out, int out_dtype, uint32_t flags, void *stream) {
    int64_t n, nb;
    int st = check_shape(rows, row_len, &n, &nb);
    if (st != FP4Q_OK) return st;
    if (flags & ~(uint32_t)FP4Q_FLAG_NO_FWHT) return FP4Q_ERR_ARG;
    if (out_dtype != FP4Q_OUT_F32 && out_dtype != FP4Q_OUT_BF16) return FP4Q_ERR_ARG;
    if (n == 0) return FP4Q_OK;
    if (!codes || !scales || !out) return FP4Q_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 8) || !aligned(out, 16)) return FP4Q_ERR_ALIGN;
    const Range o = rng(out, (out_dtype == FP4Q_OUT_F32 ? 4 : 2) * n);
    if (overlap(o, rng(codes, n / 2)) || overlap(o, rng(scales, n / 32))) return FP4Q_ERR_ARG;
    void *args[] = {&codes, &scales, &nb, &out};
    const bool fw = !(flags & FP4Q_FLAG_NO_FWHT), bf = out_dtype == FP4Q_OUT_BF16;
    const void *fn = fw ? (bf ? (const void *)&decompress_mx_kernel<true, true>
                              : (const void *)&decompress_mx_kernel<true, false>)
                        : (bf ? (const void *)&decompress_mx_kernel<false, true>
                              : (const void *)&decompress_mx_kernel<false, false>);
    return launch(fn, nb, kReceiverWaves, args, stream);
}

const char *fp4q_status_str(int status) {
    switch (status) {
        case FP4Q_OK: return "ok";
        case FP4Q_ERR_NULL: return "null pointer";
        case FP4Q_ERR_SHAPE: return "bad shape (rows >= 0, row_len > 0 and a multiple of 256)";
        case FP4Q_ERR_ALIGN: return "misaligned pointer (16 bytes; 4 for scales)";
        case FP4Q_ERR_K: return "peer count outside 1..16 (0..16 with a local slice)";
        case FP4Q_ERR_ARG: return "bad flags, output type, or overlapping buffers";
        case FP4Q_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
