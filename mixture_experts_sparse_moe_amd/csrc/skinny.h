// A 32-row product streamed through LDS: C[32, 32 NBLK] = A[32, K] B[32 NBLK, K]^T
// on v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulation).  Shared by the
// router (32 tokens x all experts) and the grouped GEMM for few rows per
// group (decode), where the weights are the stream.
//
// One workgroup of 4 waves.  K goes in chunks of 64 elements: the chunk of the
// 32 A rows and of the 32 NBLK B rows is fetched by direct-to-LDS DMA into one
// of NST stage buffers, NST - 1 chunks ahead of the one being multiplied, one
// barrier per chunk.  LDS rows are 128 bytes with 16-byte chunks XOR-swizzled
// (c ^ swz(row)).  The DMA instructions are unconditional: chunks past the end
// repeat the last one, into buffers that are never read.  The walk over the
// chunks may start at any chunk `rot` and wrap around.
//
// Waves and blocks (32 B rows each): the 4 waves form NG = 4 / KS groups; the
// KS waves of a group split the four 16-wide K steps of every chunk and each
// holds partial sums of the group's BPW = NBLK / NG blocks: block i of group
// gi is gi BPW + i, or gi + NG i when PAIRED (so one wave holds the same
// columns of both halves of B, e.g. gate and up rows).  The caller adds the
// partial tiles of a group's waves.
#pragma once

#include "device_util.h"

namespace moe {

constexpr int kSkChunk = 64;            // K elements per stage

// NA: A blocks of 32 rows (the router's 64-token tiles take 2; each wave then
// holds NA x BPW accumulator tiles, acc[ia * BPW + i]).
template <int NBLK_, int NST_ = (NBLK_ >= 8 ? 3 : 4), int KS_ = (NBLK_ >= 4 ? 1 : 4 / NBLK_), int NA_ = 1>
struct SkinnyShape {
    static constexpr int NBLK = NBLK_, NST = NST_, KS = KS_, NA = NA_;
    static constexpr int XS = NA * 32 * kSkChunk;              // A stage (elements)
    static constexpr int WS = NBLK * 32 * kSkChunk;            // B stage (elements)
    static constexpr int NG = 4 / KS;                          // wave groups
    static constexpr int BPW = NBLK / NG;                      // blocks per wave
    static constexpr int NS = 4 / KS;                          // K steps per wave per chunk
    static constexpr int P = NA + NBLK;                        // DMA instructions per wave per chunk
    static_assert(NST >= 3 && NST <= 4 && KS * NG == 4 && BPW * NG == NBLK, "shape");
    static_assert(NA == 1 || KS == 1, "two A blocks: whole K steps per wave");
};

// Block i of wave w.
template <class Sh, bool PAIRED>
__device__ __forceinline__ int skinny_block(int w, int i) {
    const int gi = w % Sh::NG;
    return PAIRED ? gi + Sh::NG * i : gi * Sh::BPW + i;
}

// B_POLICY: cache policy operand of the B loads (2, non-temporal, for a
// stream of weights read once: the decode GEMMs, whose gate/up took 0.324 ->
// 0.287 ms with it; 0 for the router, whose workgroups all re-read W_r from
// the L2 and lost 6 % with nt).
// src[ia], ia < NA: this lane's A row 32 ia + 8 w + lane / 8 at its swizzled
// 16-byte chunk, in the first chunk of the K range; src[j], j >= NA: B row
// 8 (w + 4 (j - NA)) + lane / 8 likewise.  Chunk c of the range is at byte offset 128 c.  Adds
// the products of nchunks chunks, walked from chunk rot (< nchunks), into
// acc.  Every wave of the workgroup must call it; on return this wave's DMAs
// have landed (other waves' only after a barrier).
template <class Sh, bool PAIRED, int B_POLICY>
__device__ __forceinline__ void skinny_mma(const char* const* src, int nchunks, int rot, uint16_t* sX0,
                                           uint16_t* sX1, uint16_t* sX2, uint16_t* sX3, uint16_t* sW0,
                                           uint16_t* sW1, uint16_t* sW2, uint16_t* sW3, f32x16_t* acc) {
    constexpr int NST = Sh::NST, BPW = Sh::BPW, P = Sh::P, NS = Sh::NS;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, r32 = lane & 31;
    const int s0 = (w / Sh::NG) * NS;   // this wave's first K step in a chunk

#define MOE_SK_DMA(sX_, sW_, st_)                                                               \
    do {                                                                                        \
        int c_ = min((st_), nchunks - 1) + rot;                                                 \
        c_ = c_ >= nchunks ? c_ - nchunks : c_;                                                 \
        const int64_t ko_ = (int64_t)c_ * (kSkChunk * 2);                                       \
        _Pragma("unroll") for (int ia = 0; ia < Sh::NA; ++ia)                                   \
            __builtin_amdgcn_global_load_lds((const void*)(src[ia] + ko_),                      \
                                             (lds_ptr_t)((sX_) + (32 * ia + 8 * w) * kSkChunk), 16, 0, 0); \
        _Pragma("unroll") for (int j = Sh::NA; j < P; ++j)                                      \
            __builtin_amdgcn_global_load_lds((const void*)(src[j] + ko_),                       \
                                             (lds_ptr_t)((sW_) + 8 * (w + 4 * (j - Sh::NA)) * kSkChunk), 16, 0, B_POLICY); \
    } while (0)

#define MOE_SK_MFMA(sX_, sW_)                                                                   \
    do {                                                                                        \
        _Pragma("unroll") for (int s_ = 0; s_ < NS; ++s_) {                                     \
            const int c_ = 2 * (s0 + s_) + half;                                                \
            bf16x8_t xa_[Sh::NA];                                                               \
            _Pragma("unroll") for (int ia = 0; ia < Sh::NA; ++ia) xa_[ia] = as_bf16x8(          \
                *reinterpret_cast<const uint4*>((sX_) + (32 * ia + r32) * kSkChunk +            \
                                                ((c_ ^ swz(32 * ia + r32)) * 8)));              \
            _Pragma("unroll") for (int i_ = 0; i_ < BPW; ++i_) {                                \
                const int r_ = skinny_block<Sh, PAIRED>(w, i_) * 32 + r32;                      \
                const bf16x8_t wb_ = as_bf16x8(*reinterpret_cast<const uint4*>(                 \
                    (sW_) + r_ * kSkChunk + ((c_ ^ swz(r_)) * 8)));                             \
                _Pragma("unroll") for (int ia = 0; ia < Sh::NA; ++ia) acc[ia * BPW + i_] =      \
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa_[ia], wb_, acc[ia * BPW + i_], 0, 0, 0); \
            }                                                                                   \
        }                                                                                       \
    } while (0)
// Chunk st_ from buffer (sX_, sW_).  When every wave is past this barrier the
// buffer of chunk st_ - 1 is free and takes chunk st_ - 1 + NST.  Issued
// chunks are consecutive, so waiting until NST - 2 chunks (of P instructions
// each) are outstanding means chunk st_ has landed.  The wait also covers the
// wave's LDS reads: a fragment read of chunk st_ - 1 still queued when the
// refill is issued could otherwise see the new data (operands that hit in
// the cache come back fast).
#define MOE_SK_STAGE(sX_, sW_, sXp_, sWp_, st_)                                                 \
    do {                                                                                        \
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0((NST - 2) * P));                            \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_SK_DMA(sXp_, sWp_, (st_) - 1 + NST);                                                \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        if ((st_) < nchunks) MOE_SK_MFMA(sX_, sW_);                                             \
    } while (0)

    MOE_SK_DMA(sX0, sW0, 0);
    MOE_SK_DMA(sX1, sW1, 1);
    if (NST > 3) MOE_SK_DMA(sX2, sW2, 2);
    for (int c = 0; c < nchunks; c += NST) {
        if (NST > 3) {
            MOE_SK_STAGE(sX0, sW0, sX3, sW3, c);
            MOE_SK_STAGE(sX1, sW1, sX0, sW0, c + 1);
            MOE_SK_STAGE(sX2, sW2, sX1, sW1, c + 2);
            MOE_SK_STAGE(sX3, sW3, sX2, sW2, c + 3);
        } else {
            MOE_SK_STAGE(sX0, sW0, sX2, sW2, c);
            MOE_SK_STAGE(sX1, sW1, sX0, sW0, c + 1);
            MOE_SK_STAGE(sX2, sW2, sX1, sW1, c + 2);
        }
    }
#undef MOE_SK_DMA
#undef MOE_SK_MFMA
#undef MOE_SK_STAGE
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));     // the repeated chunks past the end
}

}  // namespace moe
