// Split-KV partial attention with a second key stream (paged MLA / DSA
// decode), for gfx950.
//
// Method: mlxcel docs, "Sparse paged decode", the DSA section.  For a visible
// token t the score is sm_scale * (q . k[t][0:Dim]) + sm_scale * (q_extra .
// k_extra[t]): the first term reads the latent part of rows of a K
// allocation whose rows are RowStride >= Dim elements wide (the latent plus
// the indexer key), the second a pool of its own (the rope keys) through the
// same page table.  There is one KV head, so every query head attends every
// token.  The latent rows k[t][0:Dim] are also the values (the latent serves
// as key and value; the output projection is applied outside).  Everything
// else -- page table, chunk ownership, base-2 scores, normalized partial rows
// with log2 LSEs -- is the decode-v2 partial (PR #984 body item 2).
//
// gfx950 mapping.  Dim = 512 and ExtraDim = 64: a token's key is 576 halves.
// A workgroup is one (chunk, q group) unit of 64 query heads, one wave per 16
// heads (a group of 16 or 32 heads leaves waves idle in the products; those
// waves still move their share of every tile).  Tiles of 32 tokens x 576
// halves are staged in LDS (two stages, the latent rows by direct-to-LDS
// loads) and shared by the waves: each key and value element is fetched from
// memory once per unit.  Per 32-token tile a
// wave computes, for each 16-token half,
//   S^T [16 tokens x 16 heads] = K [16 x 576] . Q^T [576 x 16]
// with 18 v_mfma_f32_16x16x32_f16 (Q^T held in registers, loaded once), then
// one softmax update over the 32 tokens and
//   O^T [512 dims x 16 heads] += V^T [512 x 32 tokens] . P^T [32 x 16 heads]
// with 2 x 32 v_mfma_f32_16x16x32_f16 (P^T as an fp16 part and an fp16
// remainder, so the weights enter the product with about 22 bits, not
// fp16's 11), V^T read from the LDS tile with the transpose read
// ds_read_b64_tr_b16.  The lane layouts are those of the
// decode-v2 MFMA kernel: a lane owns one head's running max and sum and 128 of
// its output dims, so a rescale is a per-lane scalar.
//
// The q groups of one chunk read the same tiles.  Workgroup ids are dealt to
// the 8 XCDs round robin, so the ids are arranged to put the q groups of a
// chunk on one XCD, where the second reader finds the tiles in its L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "pd_device.h"
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kDim = 512;                     // latent: keys and values
constexpr int kExtra = 64;                    // second key stream
constexpr int kKey = kDim + kExtra;           // key halves per token
constexpr int kPieces = kKey / 8;             // 16-byte pieces per token (64 latent + 8 extra)
constexpr int kTile = 32;                     // tokens per LDS stage
constexpr int kRowBytes = kKey * 2;           // LDS row: 1152 bytes, 9 blocks of 128

// LDS swizzle.  Piece c (16 bytes) of row j is stored at piece c ^ swz(j),
// i.e. permuted within its 128-byte block, with
//   swz(j) = 2*s(j) + (j/2)%2,  s(j) = ((j/4)%4) ^ (3*((j/2)%2)).
// Rows are 1152 bytes.  The 32-byte slot s(j) differs between the four rows
// of every j%4 class and, for a fixed (j/4)%4, between rows j and j+2; the
// low bit separates the rows that share a slot.  Measured on MI355X with a
// read-only LDS microbenchmark (8 waves per CU): the key fragment reads
// (16 rows, one 16-byte piece each, per 16-lane group) run at the rate of
// lane-contiguous 16-byte reads, 5.5 clocks per instruction per CU, where the
// previous swizzle 2*((j/2)%4) + (j/8)%2 took 8.4; the value transpose reads
// run at the lane-contiguous rate under both.
__device__ __forceinline__ int swz_slot(int j) { return ((j >> 2) & 3) ^ (3 * ((j >> 1) & 1)); }
__device__ __forceinline__ int swz(int j) { return 2 * swz_slot(j) + ((j >> 1) & 1); }
constexpr int kXcds = 8;
constexpr int kWaves = 4;
constexpr int kGroupHeads = 16 * kWaves;      // query heads per workgroup
constexpr int kOffRing = 4;                   // tiles of row offsets kept (three ahead)
#ifndef PD_MLA_KEY_AHEAD
#define PD_MLA_KEY_AHEAD 3
#endif
#ifndef PD_MLA_VALUE_AHEAD
#define PD_MLA_VALUE_AHEAD 6
#endif
constexpr int kKeyAhead = PD_MLA_KEY_AHEAD;   // key steps whose LDS reads run ahead of the products
constexpr int kValueAhead = PD_MLA_VALUE_AHEAD;   // value steps likewise
// P^T enters the value product as an fp16 part plus an fp16 remainder
// (two products per value step), so the weights keep about 22 bits instead
// of fp16's 11
constexpr bool kSplitP = true;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kMfma = 0x008;
constexpr int kDsRead = 0x100;
constexpr float kMlaNoMax = -1e30f;           // finite "no score yet" running max
constexpr float kMlaLazyMargin = 8.0f;        // log2 units: p <= 2^8 between rescales

// 16 zero bytes in device memory: the source of every masked piece (tokens
// past the chunk, tiles past the last), so that all loads of the pipeline are
// unconditional and masked rows reach LDS as zeros
__device__ __align__(16) uint4 g_zero16 = {0u, 0u, 0u, 0u};

// One direct-to-LDS load: lane l's 16 bytes at src go to LDS byte address
// lds + 16*l (lds wave-uniform).  Written as inline assembly so that the
// compiler does not treat every later LDS read as waiting for it (it cannot
// tell the stage being filled from the one being read and would wait for
// all loads in flight before the first read).  The compiler does not count
// these loads in its own waits; that only makes its waits for other loads
// longer (the counter is in order), never shorter.  The caller waits for
// them (wait_loads) before the barrier that publishes the stage.
__device__ __forceinline__ void dma16(const char *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
// s_waitcnt vmcnt(0), leaving the other counters alone
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0xF70); }

struct MlaArgs {
    const _Float16 *q;      // [B, Hq, 512]
    const _Float16 *qx;     // [B, Hq, 64]
    const char *k;          // latent rows (bytes)
    const char *x;          // second-stream rows (bytes)
    int64_t k_page_stride, k_token_stride, x_page_stride, x_token_stride;   // elements
    const int32_t *indices, *indptr, *lpl, *fpo, *req_idx, *tile_idx;
    int32_t num_chunks, num_qo_heads, page_size, pages_per_chunk, q_groups;
    FastDiv fd;
    float scale_log2;
    float *v_out;           // [N, Hq, 512]
    float *lse_out;         // [N, Hq]
};

__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_partial_kernel(MlaArgs a)
{
    constexpr int NT = 64 * kWaves;

    __shared__ __align__(16) char s_tile[2][kTile * kRowBytes];
    __shared__ int64_t s_koff[kOffRing][kTile];   // byte offset of a token's rows; -1 = masked
    __shared__ int64_t s_xoff[kOffRing][kTile];

    // workgroup id -> (chunk, q group); the q groups of a chunk share id mod 8
    const int qgs = a.q_groups;
    const int b = blockIdx.x;
    const int blk = b / (kXcds * qgs);
    const int rem = b - blk * kXcds * qgs;
    const int qg = rem / kXcds;
    const int n = blk * kXcds + (rem - qg * kXcds);
    if (n >= a.num_chunks) return;                // padding of the id space

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int col = lane & 15;

    const int r = ld_uniform(a.req_idx + n);
    const int t = ld_uniform(a.tile_idx + n);
    const int pbeg = ld_uniform(a.indptr + r);
    const int npages = ld_uniform(a.indptr + r + 1) - pbeg;
    const int fpo = ld_uniform(a.fpo + r);
    const int lpl = ld_uniform(a.lpl + r);
    const int ps = a.page_size;
    const int64_t n_r = npages > 0 ? int64_t(npages - 1) * ps + lpl - fpo : 0;
    const int64_t span = int64_t(a.pages_per_chunk) * ps;
    const int64_t tok0 = max(int64_t(0), int64_t(t) * span - fpo);
    const int64_t tok1 = min(n_r, int64_t(t + 1) * span - fpo);
    const int ntok = tok1 > tok0 ? int(tok1 - tok0) : 0;
    const int ntiles = (ntok + kTile - 1) / kTile;

    const int head0 = qg * kGroupHeads + wave * 16;     // the wave's first head
    const bool active = head0 < a.num_qo_heads;         // wave-uniform (groups of 16)
    const int head = head0 + col;

    // Q^T operand of the score product, loaded once into registers: lane l
    // holds head l%16 of the wave (clamped to the last head in a short
    // group), key dims 32*kc + 8*(l/16) .. + 7 for every key step kc -- the
    // latent dims from q, the last two steps from q_extra.  Issued before
    // the page ids so that both latencies overlap.
    constexpr int KS = kPieces / 4;                        // 18 key steps
    half8_t qf[KS];
    {
        const int64_t qrow = int64_t(r) * a.num_qo_heads + min(head, a.num_qo_heads - 1);
#pragma unroll
        for (int kc = 0; kc < KS; ++kc) {
            const int d = 32 * kc + 8 * grp;
            qf[kc] = kc < kDim / 32
                ? *reinterpret_cast<const half8_t *>(a.q + qrow * kDim + d)
                : *reinterpret_cast<const half8_t *>(a.qx + qrow * kExtra + (d - kDim));
        }
    }

    // Row ids and byte offsets.  Every load of the pipeline is issued
    // unconditionally (a masked piece reads the zero block), so the compiler's
    // wait counts before each use of a register it loads cover exactly the
    // loads that use waits for.
    //
    // Page id of token tid % 32 of tile i (clamped into the request's pages;
    // tiles past the chunk load a valid id that is never used).
    auto load_id = [&](int i) -> int32_t {
        const int64_t tok = min(tok0 + int64_t(i) * kTile + (tid & (kTile - 1)), tok1 - 1);
        const uint32_t pg = fastdiv_q(a.fd, uint32_t(fpo + max(tok, int64_t(0))));
        return a.indices[pbeg + min(int64_t(pg), int64_t(npages - 1))];
    };
    // byte offsets of tile i's rows from its ids (one thread per token), kept
    // in slot i % kOffRing; -1 marks a token outside the chunk
    auto offsets = [&](int i, int32_t row) {
        const int buf = i % kOffRing;
        if (tid < kTile) {
            const int64_t tok = tok0 + int64_t(i) * kTile + tid;
            int64_t ko = -1, xo = -1;
            if (tok < tok1) {
                const uint32_t slot = uint32_t(fpo + tok);
                const uint32_t pg = fastdiv_q(a.fd, slot);
                const int64_t e = int64_t(slot - pg * uint32_t(ps));
                ko = (int64_t(row) * a.k_page_stride + e * a.k_token_stride) * 2;
                xo = (int64_t(row) * a.x_page_stride + e * a.x_token_stride) * 2;
            }
            s_koff[buf][tid] = ko;
            s_xoff[buf][tid] = xo;
        }
    };
    // Moving a tile.  The latent rows go from memory straight into LDS with
    // direct-to-LDS loads (global_load_lds_dwordx4): one instruction moves a
    // whole 1024-byte row, lane l's 16 bytes landing at byte 16*l of the row
    // in LDS, so lane l loads the piece that the swizzle puts there, piece
    // l ^ swz(j).  Wave w moves rows w + 4*k (k < 8).  The rope keys (128
    // bytes per row, not contiguous between rows in LDS) go through a
    // register: thread t moves piece t % 8 of row t / 8, loaded one
    // iteration before it is written.  Each wave waits for its direct-to-LDS
    // loads before the barrier that follows them; a stage is read only after
    // that barrier.
    constexpr int kLatRowsPerWave = kTile / kWaves;               // 8
    static_assert(kTile * (kExtra / 8) == NT, "tile / thread layout");
    const int ext_c = tid & 7;
    const int ext_r = tid >> 3;
    const char *zero = reinterpret_cast<const char *>(&g_zero16);
    typedef __attribute__((address_space(3))) char lds_char;
    auto dma_latent = [&](int i) {
        const int buf = i % kOffRing;
        const bool live = i < ntiles;
        // all row offsets first: each load is a volatile statement that the
        // compiler keeps in order with every memory access
        int64_t off[kLatRowsPerWave];
#pragma unroll
        for (int k = 0; k < kLatRowsPerWave; ++k) off[k] = s_koff[buf][wave + kWaves * k];
        const uint32_t t = __builtin_amdgcn_readfirstlane(
            uint32_t(uintptr_t((lds_char *)s_tile[i & 1])));
#pragma unroll
        for (int k = 0; k < kLatRowsPerWave; ++k) {
            const int j = wave + kWaves * k;
            const char *src = live && off[k] >= 0 ? a.k + off[k] + 16 * (lane ^ swz(j)) : zero;
            dma16(src, t + uint32_t(j * kRowBytes));
        }
    };
    auto load_rope = [&](int i) -> uint4 {
        const int64_t xo = s_xoff[i % kOffRing][ext_r];
        return load_nt(i < ntiles && xo >= 0 ? a.x + xo + 16 * ext_c : zero);
    };
    auto store_rope = [&](const uint4 &v, int buf) {
        *reinterpret_cast<uint4 *>(s_tile[buf] + ext_r * kRowBytes +
                                   16 * ((kDim / 8 + ext_c) ^ swz(ext_r))) = v;
    };

    float m_run = kMlaNoMax;          // running max of this lane's head
    float l_part = 0.f;               // this lane's share of its head's sum
    float4_t acc[kDim / 16];          // O^T: dims 16*dt + 4*(l/16) + i of head l%16
#pragma unroll
    for (int dt = 0; dt < kDim / 16; ++dt) acc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};

    typedef __attribute__((address_space(3))) short4_t lds_short4;
    // transpose-read address of a 4-token x 16-dim block: row 4*(l/16) +
    // (l%16)/4 of the subtile, halves 4*(l%4) of the dim block
    //
    // With the swizzle, lane l's read of row j = 4*g + r (g = l/16, r =
    // (l%16)/4) at halves 16*dt + 4*(l%4), i.e. piece 2*dt + (l%4)/2, is at
    // piece 2*((dt%4) ^ s(j)) + ((l%4)/2 ^ (r/2)) + 8*(dt/4), with s(j) =
    // g ^ (3*(r/2)): one base per value of dt % 4, plus 32 * (dt - dt % 4)
    // bytes.
    const int tr_r = col >> 2;
    const int tr_s = grp ^ (3 * (tr_r >> 1));
    int tr_base[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        tr_base[d] = (4 * grp + tr_r) * kRowBytes + 32 * (d ^ tr_s) +
                     16 * (((lane & 3) >> 1) ^ (tr_r >> 1)) + 8 * (lane & 1);

    // One tile: S^T for both 16-token subtiles, one softmax update over its
    // 32 tokens, then O^T += V^T . P^T as 2 x 32 products with K = 32 tokens
    // (the fp16 part of P^T and its remainder).  The
    // k order of the value product is the score layout's: lane l holds
    // tokens 4*(l/16) + e of subtile 0 as k = 8*(l/16) + e and tokens
    // 16 + 4*(l/16) + e as k = 8*(l/16) + 4 + e, so P^T needs no data
    // movement and V^T is two transpose reads, one per subtile.
    auto compute = [&](int i, int buf) {
        const char *tile = s_tile[buf];
        // key fragment kc of lane l is piece (4*kc + l/16) ^ swz(l%16)
        // = 4*(kc ^ sb) + (l/16 ^ (swz & 3)), sb = swz / 4: the bases for even
        // and odd kc differ
        const int sw = swz(col);
        const int sb = sw >> 2;
        const int lo = 16 * (grp ^ (sw & 3));
        const char *kr_even = tile + col * kRowBytes + lo + 64 * sb;
        const char *kr_odd = tile + col * kRowBytes + lo - 64 * sb;
        float4_t sc0 = float4_t{0.f, 0.f, 0.f, 0.f};
        float4_t sc1 = float4_t{0.f, 0.f, 0.f, 0.f};
        // Fragment reads run ahead of the products (kKeyAhead key steps,
        // kValueAhead value steps), so each product waits for a read issued
        // well before it: one wave per SIMD has no other wave to cover LDS
        // latency.
        auto kfrag = [&](int kc, half8_t &k0, half8_t &k1) {
            const char *kr = (kc & 1) ? kr_odd : kr_even;
            k0 = *reinterpret_cast<const half8_t *>(kr + 64 * kc);
            k1 = *reinterpret_cast<const half8_t *>(kr + 16 * kRowBytes + 64 * kc);
        };
        constexpr int KD = kKeyAhead + 1;                  // key fragment ring
        half8_t fk0[KD], fk1[KD];
#pragma unroll
        for (int kc = 0; kc < KD - 1; ++kc) kfrag(kc, fk0[kc], fk1[kc]);
#pragma unroll
        for (int kc = 0; kc < KS; ++kc) {
            if (kc + KD - 1 < KS)
                kfrag(kc + KD - 1, fk0[(kc + KD - 1) % KD], fk1[(kc + KD - 1) % KD]);
            sc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fk0[kc % KD], qf[kc], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fk1[kc % KD], qf[kc], sc1, 0, 0, 0);
        }
        // the issue order the scheduler must keep: kKeyAhead steps of reads,
        // then two products and one step of reads per step
        __builtin_amdgcn_sched_group_barrier(kDsRead, 2 * kKeyAhead, 0);
#pragma unroll
        for (int kc = 0; kc < KS - kKeyAhead; ++kc) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kMfma, 2 * kKeyAhead, 0);
        float x[8];
        float mb = -INFINITY;
        const int base = i * kTile + 4 * grp;             // chunk-relative token of e = 0
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = base + e < ntok ? sc0[e] * a.scale_log2 : -INFINITY;
            x[4 + e] = base + 16 + e < ntok ? sc1[e] * a.scale_log2 : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) mb = fmaxf(mb, x[e]);
        mb = group_max4(mb);                               // over the tile's 32 tokens
        const bool need = mb > m_run + kMlaLazyMargin;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = need ? mb : m_run;
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_part *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDim / 16; ++dt) acc[dt] *= alpha;
        }
        // P^T as the B operand: p rounded to fp16 (pb) and, with kSplitP, the
        // rounding's remainder rounded to fp16 (pl), each taken by its own
        // value product; the sum takes the weights the products use
        half8_t pb, pl;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(x[e] - m_run);
            const _Float16 ph = _Float16(p);
            pb[e] = ph;
            if constexpr (kSplitP) {
                pl[e] = _Float16(p - float(ph));
                ls += p;
            } else {
                ls += float(ph);
            }
        }
        l_part += ls;
        auto vfrag = [&](int dt) -> half8_t {
            const char *vd = tile + tr_base[dt & 3] + 32 * (dt & ~3);
            const half4_t v0 = __builtin_bit_cast(
                half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)vd));
            const half4_t v1 = __builtin_bit_cast(
                half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                             (lds_short4 *)(vd + 16 * kRowBytes)));
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int VS = kDim / 16;                      // 32 value steps
        // The remainder's product for step dt is issued two steps later, so
        // it does not wait on the same accumulator's previous product; the
        // fragment ring keeps those two steps' fragments.
        constexpr int kLag = kSplitP ? 2 : 0;
        constexpr int VD = kValueAhead + 1 + kLag;         // value fragment ring
        half8_t fv[VD];
#pragma unroll
        for (int dt = 0; dt < kValueAhead; ++dt) fv[dt] = vfrag(dt);
#pragma unroll
        for (int dt = 0; dt < VS; ++dt) {
            if (dt + kValueAhead < VS) fv[(dt + kValueAhead) % VD] = vfrag(dt + kValueAhead);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fv[dt % VD], pb, acc[dt], 0, 0, 0);
            if constexpr (kSplitP) {
                if (dt >= kLag)
                    acc[dt - kLag] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        fv[(dt - kLag) % VD], pl, acc[dt - kLag], 0, 0, 0);
            }
        }
        if constexpr (kSplitP) {
#pragma unroll
            for (int dt = VS - kLag; dt < VS; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fv[dt % VD], pl, acc[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kDsRead, 2 * kValueAhead, 1);
#pragma unroll
        for (int dt = 0; dt < kLag; ++dt) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 1);
        }
#pragma unroll
        for (int dt = kLag; dt < VS - kValueAhead; ++dt) {
            __builtin_amdgcn_sched_group_barrier(kMfma, kSplitP ? 2 : 1, 1);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(kMfma, kSplitP ? 2 * kValueAhead + kLag : kValueAhead,
                                             1);
    };

    // Pipeline.  Before iteration i: LDS stage i%2 holds tile i, the rope
    // register holds tile i+1's rope piece (loaded in the previous
    // iteration) and the offsets of tiles i+1 and i+2 are in their slots.
    // Iteration i writes tile i+1's rope piece into stage (i+1)%2 (last read
    // by tile i-1, before the previous barrier), starts its latent rows into
    // the same stage, loads tile i+2's rope piece and tile i+3's ids,
    // computes tile i, writes tile i+3's offsets and ends with the one
    // barrier, before which the kernel waits for tile i+1's loads.  The loop
    // is not unrolled: one copy of the rare rescale path keeps the compiler
    // from moving accumulator copies into the body.  Past the chunk the
    // offsets are -1 and the loads read zeros, written to a stage no later
    // tile reads.
    if (ntiles > 0) {
        offsets(0, load_id(0));
        offsets(1, load_id(1));
        offsets(2, load_id(2));
        __syncthreads();
        dma_latent(0);
        store_rope(load_rope(0), 0);
        uint4 rope = load_rope(1);
        wait_loads();
        __syncthreads();
#pragma clang loop unroll(disable)
        for (int i = 0; i < ntiles; ++i) {
            store_rope(rope, (i + 1) & 1);     // before the loads into the same stage,
            dma_latent(i + 1);                 // which the compiler would otherwise wait for
            rope = load_rope(i + 2);
            const int32_t id = load_id(i + 3);
            if (active) compute(i, i & 1);
            offsets(i + 3, id);
            wait_loads();                      // tile i+1's rows, before the barrier publishes them
            __syncthreads();
        }
    }

    if (!active) return;
    // head sum over the four 16-lane groups; each group holds 4 of every 16
    // dims, so the accumulators need no combine
    const float l = group_sum4(l_part);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *vrow = a.v_out + (int64_t(n) * a.num_qo_heads + head) * kDim + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < kDim / 16; ++dt) {
        const float4_t o = acc[dt] * inv;
        *reinterpret_cast<float4 *>(vrow + 16 * dt) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (grp == 0)
        a.lse_out[int64_t(n) * a.num_qo_heads + head] = l > 0.f ? m_run + fast_log2(l) : -INFINITY;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Query heads one MLA workgroup serves, or a negative code if the group is
// not supported.
int mla_q_heads_per_wg(int32_t num_qo_heads)
{
    if (num_qo_heads != 16 && num_qo_heads != 32 && num_qo_heads != 64 && num_qo_heads != 128)
        return fail(PD_E_UNSUPPORTED, "paged MLA decode: query heads must be 16, 32, 64 or 128");
    return num_qo_heads < kGroupHeads ? num_qo_heads : kGroupHeads;
}

// Resident MLA workgroups on `device` (CUs x workgroups per CU).
int mla_resident_wgs(int32_t device, int32_t num_qo_heads)
{
    const int qh = mla_q_heads_per_wg(num_qo_heads);
    if (qh < 0) return qh;
    int dev = device;
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess)
        return fail(PD_E_HIP, "paged MLA decode: no current device");
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(PD_E_HIP, "paged MLA decode: cannot query CU count");
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
        return fail(PD_E_HIP, "paged MLA decode: cannot select device");
    int per_cu = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(mla_partial_kernel), 64 * kWaves, 0);
    if (prev >= 0 && prev != dev && hipSetDevice(prev) != hipSuccess)
        return fail(PD_E_HIP, "paged MLA decode: cannot restore device");
    if (e != hipSuccess || per_cu < 1)
        return fail(PD_E_HIP, "paged MLA decode: occupancy query failed");
    return cus * per_cu;
}

}  // namespace pd

using namespace pd;

extern "C" int paged_mla_decode_partial(
    const void *q, const void *q_extra, const void *k_pool, const void *k_extra_pool,
    int64_t k_page_stride, int64_t k_token_stride, int64_t x_page_stride,
    int64_t x_token_stride, int32_t dim, int32_t extra_dim, int32_t dtype,
    const int32_t *indices, const int32_t *indptr, const int32_t *last_page_len,
    const int32_t *first_page_offset, const int32_t *request_indices,
    const int32_t *kv_tile_indices, int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
    int32_t num_qo_heads, int32_t page_size, float sm_scale, float *v_partial,
    float *lse_partial, void *stream)
{
    if (!q || !q_extra || !k_pool || !k_extra_pool || !indices || !indptr || !last_page_len ||
        !first_page_offset || !request_indices || !kv_tile_indices || !v_partial || !lse_partial)
        return fail(PD_E_NULL, "paged_mla_decode_partial: null pointer");
    if (num_chunks < 0 || pages_per_chunk < 1 || batch < 1 || page_size < 1 || num_qo_heads < 1 ||
        !(sm_scale > 0.f))
        return fail(PD_E_ARG, "paged_mla_decode_partial: bad sizes");
    if (dtype != PD_DTYPE_FP16 || dim != kDim || extra_dim != kExtra)
        return fail(PD_E_UNSUPPORTED,
                    "paged_mla_decode_partial: only fp16 with dim 512 and extra_dim 64");
    const int qh = mla_q_heads_per_wg(num_qo_heads);
    if (qh < 0) return qh;
    if (!aligned16(q) || !aligned16(q_extra) || !aligned16(k_pool) || !aligned16(k_extra_pool) ||
        (k_page_stride * 2) % 16 || (k_token_stride * 2) % 16 || (x_page_stride * 2) % 16 ||
        (x_token_stride * 2) % 16 || k_page_stride < 0 || k_token_stride < 0 ||
        x_page_stride < 0 || x_token_stride < 0)
        return fail(PD_E_UNSUPPORTED,
                    "paged_mla_decode_partial: pools and queries must be 16-byte aligned");
    if (num_chunks == 0) return PD_OK;
    if (num_chunks > PD_MAX_CHUNKS)
        return fail(PD_E_ARG, "paged_mla_decode_partial: too many chunks");
    MlaArgs a;
    a.q = static_cast<const _Float16 *>(q);
    a.qx = static_cast<const _Float16 *>(q_extra);
    a.k = static_cast<const char *>(k_pool);
    a.x = static_cast<const char *>(k_extra_pool);
    a.k_page_stride = k_page_stride;
    a.k_token_stride = k_token_stride;
    a.x_page_stride = x_page_stride;
    a.x_token_stride = x_token_stride;
    a.indices = indices;
    a.indptr = indptr;
    a.lpl = last_page_len;
    a.fpo = first_page_offset;
    a.req_idx = request_indices;
    a.tile_idx = kv_tile_indices;
    a.num_chunks = num_chunks;
    a.num_qo_heads = num_qo_heads;
    a.page_size = page_size;
    a.pages_per_chunk = pages_per_chunk;
    a.q_groups = (num_qo_heads + kGroupHeads - 1) / kGroupHeads;
    a.fd = make_fastdiv(uint32_t(page_size));
    a.scale_log2 = float(double(sm_scale) * 1.4426950408889634);
    a.v_out = v_partial;
    a.lse_out = lse_partial;
    const int64_t blocks = (int64_t(num_chunks) + kXcds - 1) / kXcds * kXcds * a.q_groups;
    hipLaunchKernelGGL(mla_partial_kernel, dim3(uint32_t(blocks)), dim3(64 * kWaves), 0,
                       static_cast<hipStream_t>(stream), a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_mla_decode_partial: launch failed: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}
