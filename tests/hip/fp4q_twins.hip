// fp4q_twins.hip -- MEASUREMENT-ONLY library: compute-free "traffic twins" of
// the library's kernels, timed beside them by bench.py (its ceilings leg).
//
// Each twin runs the same launch shape (tiles, wavefronts per workgroup, LDS
// region) and issues the same memory instructions as the kernel it mirrors --
// it calls the kernel's own load and store functions -- but replaces the
// transform and quantisation arithmetic by a few integer operations on the
// loaded words.  Its time is therefore what that exact traffic pattern costs
// on the memory system, the ceiling the kernel can approach.  Two plain
// streams give the read-only and write-only rates for reference.
//
// Every load and store stays inside the buffers the kernels themselves use
// (the same bounds logic); the host functions check sizes like the library.
#include "fp4q.hip"

namespace {

// Folds the loaded words of a lane into its 64 registers (no arithmetic on the
// values, one integer operation per register).
__device__ __forceinline__ void fill_registers(const unsigned (&w)[8], unsigned salt, float (&R)[64]) {
#pragma unroll
    for (int j = 0; j < 64; ++j) R[j] = as_f(w[j & 7] ^ (salt + (unsigned)j));
}

// decompress_kernel<true, kBf16>'s traffic: its payload loads and its output,
// staged through LDS as the kernel stages it (fp32 in rounds, bf16 at once).
template <bool kBf16>
__global__ __launch_bounds__(kWave * kDecompressWaves<kBf16>) void twin_decompress_kernel(
    const uint4 *__restrict__ codes, const uint4 *__restrict__ micro, const float *__restrict__ block,
    int64_t nblocks, void *__restrict__ out) {
    __shared__ uint4 lds[kDecompressWaves<kBf16> * kReceiverChunks<kBf16>];
    const Lane L = lane_map<kDecompressWaves<kBf16>>(nblocks);
    uint4 *wl = lds + (threadIdx.x / kWave) * kReceiverChunks<kBf16>;
    const PayloadRegs P = load_payload(L, codes, micro, block);
    const unsigned w[8] = {P.c0.x, P.c0.y, P.c0.z, P.c0.w, P.c1.x, P.c1.y, P.c1.z, P.c1.w};
    float R[64];
    fill_registers(w, P.lo ^ P.hi ^ as_u(P.s), R);
    store_out<kBf16, kStreamPolicy<true>>(L, nblocks, wl, out, R);
}

// accumulate_narrow_kernel<true, false>'s traffic: k payloads loaded as the
// narrow layout loads them (one contiguous 1 KiB of codes per peer, a 2-byte
// micro-scale pair and the block scale per lane), then the fp32 output through
// LDS in the same two rounds.
__global__ __launch_bounds__(kWave * kReceiverWaves) void twin_accumulate_kernel(
    Peers peers, int k, int64_t nblocks, float *__restrict__ out) {
    __shared__ uint4 lds[kReceiverWaves * kNarrowOutChunks];
    const NarrowLane L = narrow_map<kReceiverWaves, true>(nblocks);
    uint4 *wl = lds + (threadIdx.x / kWave) * kNarrowOutChunks;
    unsigned w[4] = {0, 0, 0, 0}, salt = 0;
    NarrowPayload P = load_narrow(L, peers.codes[0], peers.micro[0], peers.block[0]);
    for (int p = 0; p < k; ++p) {
        const NarrowPayload cur = P;
        if (p + 1 < k) P = load_narrow(L, peers.codes[p + 1], peers.micro[p + 1], peers.block[p + 1]);
        w[0] ^= cur.c.x;
        w[1] ^= cur.c.y;
        w[2] ^= cur.c.z;
        w[3] ^= cur.c.w;
        salt ^= cur.m ^ as_u(cur.s);
    }
    float R[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) R[j] = as_f(w[j & 3] ^ (salt + (unsigned)j));
    narrow_store_out<false>(L, nblocks, wl, out, R);
}

// compress_kernel<true>'s traffic: the bf16 tile through LDS as load_widen
// stages it, then the codes through LDS and the micro- and block-scale stores.
__global__ __launch_bounds__(kWave * kSenderWaves) void twin_compress_kernel(
    const uint4 *__restrict__ in, int64_t nblocks, uint4 *__restrict__ codes,
    unsigned *__restrict__ micro, float *__restrict__ block) {
    __shared__ uint4 lds_all[kSenderWaves * kStageChunks];
    const Lane L = lane_map<kSenderWaves>(nblocks);
    uint4 *lds = lds_all + (threadIdx.x / kWave) * kStageChunks;
    {
        uint4 d[8];
        load_tile(in, L.tile, nblocks, L.lane, d);
        uint4 *dst = lds + 33 * (L.lane >> 5) + (L.lane & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[66 * j] = d[j];
    }
    wave_lds_sync();
    unsigned C[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint4 *srcl = lds + 33 * L.p + 8 * L.q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 x = srcl[i];
        C[i] = x.x ^ x.y ^ x.z ^ x.w;
    }
    wave_lds_sync();  // every lane has read its chunks from the region
    store_codes<kStreamPolicy<true>>(L, nblocks, lds, codes, C);
    if (L.valid) {
        TileStore(micro, L.tile, nblocks, 16).b32(16 * L.p + 4 * L.q, C[0] ^ C[5]);
        if (L.q == 0) TileStore(block, L.tile, nblocks, 4).b32(4 * L.p, C[1] ^ C[7]);
    }
}

// Plain streams over nbytes (a multiple of 16 KiB): every wavefront moves
// 16 KiB as sixteen 1 KiB instructions, loads on the non-temporal path (all
// folded into one 16-byte store per wavefront) or stores with the library's
// policy.
__global__ __launch_bounds__(256) void twin_read_kernel(const uint4 *__restrict__ in, int64_t nwaves,
                                                        uint4 *__restrict__ sink) {
    const int64_t wv = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (wv >= nwaves) return;
    const int lane = threadIdx.x & (kWave - 1);
    const uint4 *src = in + wv * 1024 + lane;
    uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint4 v = load_nt(src + 64 * j);
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    // every lane's loads feed the stored word (a store by one lane alone would
    // let the compiler move the other lanes' loads under its branch)
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        acc.x ^= (unsigned)__shfl_xor((int)acc.x, m);
        acc.y ^= (unsigned)__shfl_xor((int)acc.y, m);
        acc.z ^= (unsigned)__shfl_xor((int)acc.z, m);
        acc.w ^= (unsigned)__shfl_xor((int)acc.w, m);
    }
    if (lane == 0) sink[wv] = acc;
}

__global__ __launch_bounds__(256) void twin_write_kernel(uint4 *__restrict__ out, int64_t nwaves) {
    const int64_t wv = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (wv >= nwaves) return;
    const int lane = threadIdx.x & (kWave - 1);
    const TileStoreP<kStreamPolicy<true>> dst(out + wv * 1024, 0, 1, 16384, 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) dst.b128(16 * (64 * j + lane), make_uint4(lane, j, 0, 0));
}

}  // namespace

extern "C" {

// The same shapes, sizes and buffers as the entry points they mirror (device
// pointers); 0 on success, -1 for bad arguments, -2 for a failed launch.
// out_dtype: FP4Q_OUT_F32 or FP4Q_OUT_BF16, as fp4q_decompress_ex.
int twin_decompress(const uint8_t *codes, const uint8_t *micro, const float *block, int64_t rows,
                    int64_t row_len, void *out, int out_dtype, void *stream) {
    int64_t n, nb;
    if (check_shape(rows, row_len, &n, &nb) != FP4Q_OK || n == 0 || !codes || !micro || !block || !out ||
        (out_dtype != FP4Q_OUT_F32 && out_dtype != FP4Q_OUT_BF16))
        return -1;
    void *args[] = {&codes, &micro, &block, &nb, &out};
    const bool bf = out_dtype == FP4Q_OUT_BF16;
    const void *fn = bf ? (const void *)&twin_decompress_kernel<true> : (const void *)&twin_decompress_kernel<false>;
    return launch(fn, nb, bf ? kDecompressWaves<true> : kReceiverWaves, args, stream) == FP4Q_OK ? 0 : -2;
}

int twin_accumulate(int k, const uint8_t *const *codes, const uint8_t *const *micro,
                    const float *const *block, int64_t rows, int64_t row_len, float *out, void *stream) {
    int64_t n, nb;
    if (check_shape(rows, row_len, &n, &nb) != FP4Q_OK || n == 0 || k < 1 || k > FP4Q_MAX_PEERS || !out)
        return -1;
    Peers peers = {};
    for (int p = 0; p < k; ++p) {
        if (!codes[p] || !micro[p] || !block[p]) return -1;
        peers.codes[p] = reinterpret_cast<const uint4 *>(codes[p]);
        peers.micro[p] = reinterpret_cast<const uint4 *>(micro[p]);
        peers.block[p] = block[p];
    }
    void *args[] = {&peers, &k, &nb, &out};
    return launch((const void *)&twin_accumulate_kernel, nb, kReceiverWaves, args, stream, kNarrowBlocks) == FP4Q_OK
               ? 0
               : -2;
}

int twin_compress(const uint16_t *in, int64_t rows, int64_t row_len, uint8_t *codes, uint8_t *micro,
                  float *block, void *stream) {
    int64_t n, nb;
    if (check_shape(rows, row_len, &n, &nb) != FP4Q_OK || n == 0 || !in || !codes || !micro || !block)
        return -1;
    void *args[] = {&in, &nb, &codes, &micro, &block};
    return launch((const void *)&twin_compress_kernel, nb, kSenderWaves, args, stream) == FP4Q_OK ? 0 : -2;
}

// nbytes: a positive multiple of 16 KiB; sink: nbytes / 1024 bytes.
int twin_read(const void *in, int64_t nbytes, void *sink, void *stream) {
    if (!in || !sink || nbytes <= 0 || nbytes % 16384) return -1;
    int64_t nwaves = nbytes / 16384;
    void *args[] = {&in, &nwaves, &sink};
    const hipError_t e = hipLaunchKernel((const void *)&twin_read_kernel, dim3((unsigned)((nwaves + 3) / 4)),
                                         dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : -2;
}

int twin_write(void *out, int64_t nbytes, void *stream) {
    if (!out || nbytes <= 0 || nbytes % 16384) return -1;
    int64_t nwaves = nbytes / 16384;
    void *args[] = {&out, &nwaves};
    const hipError_t e = hipLaunchKernel((const void *)&twin_write_kernel, dim3((unsigned)((nwaves + 3) / 4)),
                                         dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : -2;
}

}  // extern "C"
