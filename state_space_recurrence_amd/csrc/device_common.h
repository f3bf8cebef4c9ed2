// device_common.h -- gfx950 device helpers shared by the ReplaySSM kernels.
//
// Lane layout used by every state-streaming kernel (P = 64 rows, N = 128
// columns of fp32 per head):
//   one wave64 owns one head; lane l = 32*hf + c reads, with one 16-byte
//   load, columns 4c..4c+3 of row 2i+hf for i = 0..31 (a whole 512-byte row
//   per 32-lane half, two rows per wave-wide load instruction: fully
//   coalesced).  A per-row partial dot product over the lane's 4 columns is
//   then reduced across the 32 lanes of the half by a reduce-scatter
//   butterfly after which lane c of half hf holds the total of row 2c+hf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

constexpr int kP = 64;
constexpr int kN = 128;
constexpr int kWave = 64;

// ----------------------------------------------------------------- inputs --
// Input element types: fp32, or bf16 carried as its 16 raw bits.
template <typename T> struct io;

template <> struct io<float> {
    using raw4 = float4;   // four elements as stored
    static __device__ __forceinline__ raw4 load_raw4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    static __device__ __forceinline__ float4 widen(raw4 r) { return r; }
    // widen() behind an optimisation fence: the result is recomputed at each
    // use instead of being kept live (trades 2 VALU ops for 4 VGPRs).
    static __device__ __forceinline__ float4 widen_here(raw4 r) {
        asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w));
        return r;
    }
    static __device__ __forceinline__ float load1(const float *p) { return *p; }
    static __device__ __forceinline__ float4 load4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    static __device__ __forceinline__ void copy1(float *dst, const float *src) { *dst = *src; }
};

template <> struct io<uint16_t> {
    using raw4 = uint2;    // four bf16 as stored
    static __device__ __forceinline__ raw4 load_raw4(const uint16_t *p) {
        return *reinterpret_cast<const uint2 *>(p);
    }
    static __device__ __forceinline__ float4 widen(raw4 u) {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
    static __device__ __forceinline__ float4 widen_here(raw4 u) {
        asm volatile("" : "+v"(u.x), "+v"(u.y));
        return widen(u);
    }
    static __device__ __forceinline__ float load1(const uint16_t *p) {
        return __uint_as_float(uint32_t(*p) << 16);
    }
    static __device__ __forceinline__ float4 load4(const uint16_t *p) {
        uint2 u = *reinterpret_cast<const uint2 *>(p);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
    static __device__ __forceinline__ void copy1(uint16_t *dst, const uint16_t *src) { *dst = *src; }
};

// ------------------------------------------------------------ state stream --
// The checkpoint is streamed once per step and is far larger than the caches
// at serving batch sizes, so its loads (and the commit's stores) carry the
// non-temporal hint: they do not displace the reused small tensors (inputs,
// buffer entries) from L2 / MALL.
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 stream_load4(const float *p) {
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void stream_store4(float *p, float4 v) {
    f4v u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<f4v *>(p));
}

// The same for 16 bytes of packed codes.
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 stream_load16(const uint4 *p) {
    const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void stream_store16(uint4 *p, uint4 v) {
    const u4v u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<u4v *>(p));
}

// Buffer-resource form of the same accesses (raw buffer, stride 0): word 3
// of the descriptor selects 32-bit data; cache-policy operand 2 is the
// non-temporal hint.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// A buffer resource over `bytes` bytes at a wave-uniform address (pinned to
// scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, int bytes) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0, bytes,
                                             kBufferRsrcWord3);
}

// Load at byte offset vo + soff: vo in a VGPR (covered by the descriptor's
// range check), soff a wave-uniform constant carried in the scalar offset
// operand, which the range check does not cover -- callers keep vo + soff
// inside the resource by construction.
__device__ __forceinline__ float4 buffer_stream_load4(__amdgpu_buffer_rsrc_t r, int vo, int soff) {
    const f4v v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, soff, kNonTemporal);
    return make_float4(v.x, v.y, v.z, v.w);
}

// Store at byte offset vo.  The whole offset is a VGPR operand (the scalar
// offset is the constant 0), so the range check covers it and, more
// importantly, the compiler's hazard model applies: a store of more than
// 64 bits of data must be followed by wait states before any VALU op may
// overwrite its data VGPRs, and LLVM waives that requirement when the
// scalar offset operand is a register.  A build that let the next
// instruction overwrite the data of a 128-bit store with an SGPR offset
// wrote wrong values for exactly that store's rows.
__device__ __forceinline__ void buffer_stream_store4(__amdgpu_buffer_rsrc_t r, int vo, float4 v) {
    const f4v u = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, vo, 0, kNonTemporal);
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// ------------------------------------------------------------- cross-lane --
// DPP controls (GCN/CDNA encoding).
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within a 16-lane row
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8 lanes
constexpr int kDppQuadRev = 0x1B;         // quad_perm [3,2,1,0]
constexpr int kDppQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppRowShl1 = 0x101;        // lane i <- lane i+1 within a row (0 past its end)
constexpr int kDppRowShl2 = 0x102;
constexpr int kDppRowShl4 = 0x104;
constexpr int kDppRowShl8 = 0x108;
constexpr int kDppWaveShl1 = 0x130;       // lane i <- lane i+1 across the wave (0 for lane 63)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One butterfly stage on pairs (v[i], v[i+H]): the partner lane holds the
// complementary half; the lane keeps index i if `up` is false, i+H if true.
template <int CTRL, int H, int NV>
__device__ __forceinline__ void rs_stage(float (&v)[NV], bool up) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        float lo = v[i] + dpp<CTRL>(v[i]);
        float hi = v[i + H] + dpp<CTRL>(v[i + H]);
        v[i] = up ? hi : lo;
    }
}

// Reduce-scatter of 32 per-lane values over the 32 lanes of each half-wave.
// On entry v[i] is lane c's partial of item i; on exit v[0] is the total of
// item c over the 32 lanes of the half.
__device__ __forceinline__ void reduce_scatter32(float (&v)[32], int lane) {
    // lane bit 4: rows (16-lane groups) 0<->1 and 2<->3 exchange through
    // v_permlane16_swap: odd rows of the first operand trade places with even
    // rows of the second, so both sides of each pair see own + partner.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 16]),
                                                  false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    rs_stage<kDppRowMirror, 8>(v, (lane & 8) != 0);
    rs_stage<kDppRowHalfMirror, 4>(v, (lane & 4) != 0);
    rs_stage<kDppQuadRev, 2>(v, (lane & 2) != 0);
    rs_stage<kDppQuadSwap1, 1>(v, (lane & 1) != 0);
}

// ---------------------------------------------------------- chunked stream --
// The 32 rows a lane touches (rows 2i+hf, i = 0..31) are streamed in 4 chunks
// of 8: chunk c holds i = c + 4m, m = 0..7.  With that order the first three
// butterfly stages (lane bits 4, 3, 2 <-> index bits 4, 3, 2 = m bits 2, 1, 0)
// close inside a chunk, leaving one value per chunk; the last two stages
// (lane bits 1, 0 <-> c bits 1, 0) combine the 4 chunk values.  The lane that
// ends with a total is the same as for reduce_scatter32: lane c of half hf
// holds row 2c + hf.
constexpr int kChunks = 4;
constexpr int kPerChunk = 8;

__device__ __forceinline__ int chunk_index(int c, int m) { return c + 4 * m; }

// Stages for lane bits 4, 3, 2 on the 8 partials of a chunk.
__device__ __forceinline__ float chunk_reduce8(float (&v)[8], int lane) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 4]),
                                                  false, false);
        v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    rs_stage<kDppRowMirror, 2>(v, (lane & 8) != 0);
    rs_stage<kDppRowHalfMirror, 1>(v, (lane & 4) != 0);
    return v[0];
}

// Stages for lane bits 1, 0 on the 4 chunk values.
__device__ __forceinline__ float chunk_combine4(float (&r)[4], int lane) {
    rs_stage<kDppQuadRev, 2>(r, (lane & 2) != 0);
    rs_stage<kDppQuadSwap1, 1>(r, (lane & 1) != 0);
    return r[0];
}

// Sum over the 16 lanes of a DPP row, result in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kDppRowMirror>(v);
    v += dpp<kDppRowHalfMirror>(v);
    v += dpp<kDppQuadRev>(v);
    v += dpp<kDppQuadSwap1>(v);
    return v;
}

// Suffix sums over lanes 0..NL-1 (NL = 16 or 32): lane i gets the sum of v
// over lanes i..NL-1 (Hillis-Steele within each row; for 32 lanes the second
// row's total is then added to the first row).  Lanes at or past NL must hold
// zeros.
template <int NL>
__device__ __forceinline__ float suffix_sum(float v, int lane) {
    static_assert(NL == 16 || NL == 32, "one or two DPP rows");
    v += dpp<kDppRowShl1>(v);
    v += dpp<kDppRowShl2>(v);
    v += dpp<kDppRowShl4>(v);
    v += dpp<kDppRowShl8>(v);
    if constexpr (NL == 32) {
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
        if (lane < 16) v += r1;
    }
    return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip; remap
// so that each XCD (and its L2) works on a contiguous range of logical
// workgroups (adjacent heads of the same slot share B/C and buffer reads).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    if (nwg % 8 != 0) return bid;
    return (bid % 8) * (nwg / 8) + bid / 8;
}

// Sticky device error bits (stored in work[batch]).
constexpr int kErrPos = 1;    // position count out of range on entry
constexpr int kErrKeep = 2;   // n_keep outside 0..T
constexpr int kErrSlot = 4;   // a call row mapped to a slot outside 0..nslots-1 (row skipped)
constexpr int kErrDup = 8;    // two rows of one call on the same slot (a race; results undefined)

}  // namespace rssm
