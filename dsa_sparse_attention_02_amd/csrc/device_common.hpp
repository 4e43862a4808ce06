// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l supplies row l%32 of A
// and column l%32 of B, each with the 8 consecutive k values 8*(l/32)..8*(l/32)+7.
// Lane l receives column l%32 of D at rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row of the 32x32 accumulator held in register i by a lane in half `half` (= lane/32)
__device__ __forceinline__ constexpr int acc_row(int i, int half)
{
    return 8 * (i >> 2) + 4 * half + (i & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// 16-byte load from a global-memory address held as an integer (the address
// space is explicit, so the compiler emits a global, not a flat, load)
__device__ __forceinline__ u32x4 load16_global(uint64_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(addr);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    f2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Copy 16 bytes per lane from global memory straight into LDS (gfx950 LDS-DMA):
// lane i of the wave writes lds_wave_base + 16*i.  The LDS base must be
// wave-uniform.  Completion is counted by vmcnt; the compiler does not track
// it for later LDS reads, so callers wait explicitly (or at a barrier).
__device__ __forceinline__ void dma16_to_lds(const void *src, SA_LDS void *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// The same copy with the non-temporal cache policy, for data read once: a
// streamed 1.2 GB read of random 16 KiB pages runs at ~6.7 TB/s with it
// against ~4.6 TB/s with the default policy on MI355X.
__device__ __forceinline__ void dma16_to_lds_stream(const void *src, SA_LDS void *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 2 /* nt */);
}

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format; the
// dword-count loads below ignore the format).
constexpr int kBufferWord3 = 0x00020000;

// Buffer resource over `bytes` bytes at `base` (wave-uniform: the resource
// lives in scalar registers).  Reads through it at or past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}

// The 16-byte-per-lane LDS-DMA copy in its buffer (MUBUF) form: each active
// lane i reads resource offset voff_i (32-bit) and writes lds_wave_base + 16*i.
// The compiler counts LDS reads exactly around this form, whereas after the
// global (FLAT-encoded) form it assumes the copy may still be pending on the
// LDS counter and waits for every LDS read in flight at each later use of one.
__device__ __forceinline__ void buf_dma16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, SA_LDS void *lds_wave_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, 0, 0, 0);
}

// The same with the non-temporal cache policy (data read once).
__device__ __forceinline__ void buf_dma16_to_lds_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, SA_LDS void *lds_wave_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, 0, 0, 2 /* nt */);
}

// s_barrier without the memory fence __syncthreads adds (which would wait for
// every LDS-DMA copy in flight); the asm memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// The same barrier after this wave's LDS reads and writes have completed
// (lgkmcnt(0)): LDS data written before it is visible to every wave after it.
// LDS-DMA copies are counted by vmcnt and waited for separately.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// An LDS address the compiler cannot trace to a __shared__ array: a copy into it
// carries no alias scope, so the compiler adds no wait for that copy before
// later reads of other buffers of the same array (ordering is then the
// caller's, through explicit vmcnt waits and barriers).
__device__ __forceinline__ SA_LDS void *opaque_lds(SA_LDS void *p)
{
    uint32_t a = (uint32_t)(uintptr_t)p;
    asm("" : "+s"(a));  // (not volatile: no scheduling barrier)
    return (SA_LDS void *)(uintptr_t)a;
}

// Min and max of v over the 32 lanes of each wave half (every lane gets them);
// lanes with valid == false are ignored.
__device__ __forceinline__ f32x2 minmax32(float v, bool valid)
{
    float mn = valid ? v : INFINITY, mx = valid ? v : -INFINITY;
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, d));
        mx = fmaxf(mx, __shfl_xor(mx, d));
    }
    return f32x2{mn, mx};
}

// p[l] + p[l ^ 32] in every lane: v_permlane32_swap of p with itself hands
// lanes 0..31 the upper half and lanes 32..63 the lower half.
__device__ __forceinline__ float add_wave_halves(float p)
{
    const uint32_t u = __float_as_uint(p);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Min and max of v over lanes 0..31 (lanes with valid == false ignored), as
// wave-uniform values: DPP butterflies within each 16-lane row (quad swaps,
// half-row mirror, row mirror), then the two row results read by v_readlane.
// The wave must run with every lane active.
__device__ __forceinline__ f32x2 minmax32_uniform(float v, bool valid)
{
    float mn = valid ? v : INFINITY, mx = valid ? v : -INFINITY;
    mn = fminf(mn, dpp_f32<0xB1>(mn));   // quad_perm [1,0,3,2]
    mx = fmaxf(mx, dpp_f32<0xB1>(mx));
    mn = fminf(mn, dpp_f32<0x4E>(mn));   // quad_perm [2,3,0,1]
    mx = fmaxf(mx, dpp_f32<0x4E>(mx));
    mn = fminf(mn, dpp_f32<0x141>(mn));  // row_half_mirror
    mx = fmaxf(mx, dpp_f32<0x141>(mx));
    mn = fminf(mn, dpp_f32<0x140>(mn));  // row_mirror
    mx = fmaxf(mx, dpp_f32<0x140>(mx));
    const float mn0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), 0));
    const float mn1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), 16));
    const float mx0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
    const float mx1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 16));
    return f32x2{fminf(mn0, mn1), fmaxf(mx0, mx1)};
}

// Order-preserving map from an fp32 score to uint32: a larger key is a larger
// score; -0 is folded into +0 first so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float f)
{
    f = f + 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Prefill over several sequences in one launch ("Day-0 Adaptation: Running
// Trillion-Parameter Models on Domestic AI Accelerators", 3.3: the prefill
// pathway; "Engineering Practices for Day-0 Adaptation of Million-Token Context
// Models on Domestic AI Chips" names multi-sequence load balance for it).  The
// rows of one launch are cut into pieces, each a run of consecutive query rows
// of one sequence.  The map travels by value in the kernel arguments, so the
// host builds it without a copy to the device.
constexpr int kMapPieces = 64;
struct SeqMap {
    int npieces;
    int first[kMapPieces + 1];  // ascending search keys: first row (top-k, attention) or first 16-row block (indexer)
    int row0[kMapPieces];       // the piece's first row, counted from the launch's first row
    int nrows[kMapPieces];
    int pos0[kMapPieces];       // position of the piece's first row in its sequence
    int bt_row[kMapPieces];     // the sequence's block-table row
};

// The piece whose key range holds `key` (wave-uniform: a search over kernel
// arguments).
__device__ inline int map_piece(const SeqMap &m, int key)
{
    int lo = 0, hi = m.npieces - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (m.first[mid] <= key) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The current token of each decode sequence written into the paged cache
// ("Engineering Practices for Day-0 Adaptation of Million-Token Context Models
// on Domestic AI Chips", Four Key Layers items 2 and 3: block-level
// incremental cache updates during decode, merged into the attention kernels'
// launches).  Sequence b's token sits at position context_lens[b] - 1; its
// latent row new_kv[b] and indexer key new_idx_k[b] go to that position's
// physical slot.  new_kv == nullptr: nothing to append.
struct AppendArgs {
    const uint16_t *new_kv;      // [batch][qk_dim]
    const uint16_t *new_idx_k;   // [batch][idx_dim]
    uint16_t *kv;                // the cache pools, written at one slot per sequence
    uint16_t *idx_k;
    const int32_t *block_table;  // [seqs][max_blocks]
    const int32_t *ctx_lens;
    int64_t num_blocks;
    int max_blocks, bs_log2, qk_dim, idx_dim;
};

// Physical row of sequence b's current token, or -1 (no token, or an unmapped
// block).
__device__ __forceinline__ int64_t append_slot(const AppendArgs &ap, int b)
{
    const int ctx = ap.ctx_lens[b];
    if (ctx <= 0) return -1;
    const int s = ctx - 1;
    const int blk = ap.block_table[(int64_t)b * ap.max_blocks + (s >> ap.bs_log2)];
    if (blk < 0 || blk >= ap.num_blocks) return -1;
    return ((int64_t)blk << ap.bs_log2) | (s & ((1 << ap.bs_log2) - 1));
}

// Sequence b's two new rows into the cache, 16 bytes per thread (threads
// tid = 0 .. nthreads-1 of the calling group; row widths are multiples of 8).
__device__ __forceinline__ void append_rows(const AppendArgs &ap, int b, int tid, int nthreads)
{
    if (!ap.new_kv) return;
    const int64_t slot = append_slot(ap, b);
    if (slot < 0) return;
    const int nkv = ap.qk_dim / 8, nik = ap.idx_dim / 8;
    for (int i = tid; i < nkv + nik; i += nthreads) {
        if (i < nkv)
            *reinterpret_cast<u32x4 *>(ap.kv + slot * ap.qk_dim + 8 * i) =
                load16(ap.new_kv + (int64_t)b * ap.qk_dim + 8 * i);
        else
            *reinterpret_cast<u32x4 *>(ap.idx_k + slot * ap.idx_dim + 8 * (i - nkv)) =
                load16(ap.new_idx_k + (int64_t)b * ap.idx_dim + 8 * (i - nkv));
    }
}

}  // namespace sa
