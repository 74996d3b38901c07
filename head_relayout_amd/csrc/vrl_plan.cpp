// Launch planning of the relayout kernels: vector width, kernel selection,
// tile geometry and the kernel arguments, from the problem and the operands'
// addresses and strides.  Pure host arithmetic, no device access; the
// C-ABI layer calls it after validating the operands.
#include "vrl_internal.h"

#include <algorithm>
#include <cstdint>

namespace vrl {
namespace {

// n / d == (n * magic) >> shift for every n < 2^31 (see div_magic in the kernels).
void magic_for(uint32_t d, uint64_t &magic, uint32_t &shift)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d)
        ++l;
    shift = 31 + l;
    magic = ((uint64_t(1) << shift) + d - 1) / d;
}

// Largest vector width (bytes) that divides every address, stride and row.
int vector_bytes(const PlanView *vs, int n, uintptr_t wire, int64_t D)
{
    uint64_t acc = uint64_t(D) * 2 | wire;
    for (int i = 0; i < n; ++i) {
        acc |= vs[i].ptr;
        acc |= uint64_t(vs[i].st) * 2;
        acc |= uint64_t(vs[i].sh) * 2;
    }
    for (int vb : {16, 8, 4})
        if (acc % uint64_t(vb) == 0)
            return vb;
    return 2;
}

// Heads per tile of the LDS transpose: the smallest divisor of Gb whose head
// rows fill at least one 128-byte line, else all Gb.
int64_t staged_heads(int64_t Gb, int64_t D)
{
    for (int64_t g = 1; g <= Gb; ++g)
        if (Gb % g == 0 && g * D * 2 >= 128)
            return g;
    return Gb;
}

}  // namespace

bool plan_launch(Op op, const Problem &pb, const PlanView *views, int nviews, uintptr_t wire,
                 int32_t cb, int32_t ce, LaunchPlan &pl, const char **why)
{
    const Problem *d = &pb;
    const int64_t G = d->H / d->P;
    const int vb = vector_bytes(views, nviews, wire, d->D);
    const int ve = vb / 2;

    pl = LaunchPlan{};
    pl.op = op;
    pl.vec_bytes = vb;
    // heads per wire row: the whole group, or one head chunk of it
    const int64_t Gb = d->chunk_heads ? G / d->C : G;
    pl.contig = true;
    for (int i = 0; i < nviews; ++i)
        if (Gb > 1 && views[i].sh != d->D)
            pl.contig = false;

    KernelArgs &a = pl.args;
    for (int i = 0; i < 3; ++i) {
        const PlanView &g = views[i < nviews ? i : 0];
        a.view_ptr[i] = reinterpret_cast<uint16_t *>(g.ptr);
        a.view_st[i] = g.st;
        a.view_sh[i] = g.sh;
    }
    a.wire = reinterpret_cast<uint16_t *>(wire);
    a.s_local = d->s_local;
    a.P = d->P;
    a.G = int32_t(G);
    a.D = d->D;
    a.C = d->C;
    a.chunk_heads = d->chunk_heads;
    a.row_heads = int32_t(Gb);

    const int64_t chunk_q = d->s_local / d->C, chunk_r = d->s_local % d->C;
    const int64_t row_vecs = Gb * d->D / ve;
    const int64_t t_max = d->chunk_heads ? d->s_local : chunk_q + (chunk_r ? 1 : 0);
    if (t_max > (int64_t(1) << 31) / row_vecs ||
        t_max * row_vecs + int64_t(kMaxTileVecs) >= (int64_t(1) << 31)) {
        *why = "a chunk is too large (2^31 vectors or more); use more chunks";
        return false;
    }
    const int64_t nvec_max = t_max * row_vecs;
    a.chunk_q = int32_t(chunk_q);
    a.chunk_r = int32_t(chunk_r);
    a.c_begin = cb;
    a.n_win = ce - cb;
    a.row_vecs = uint32_t(row_vecs);
    a.head_vecs = uint32_t(d->D / ve);
    magic_for(a.row_vecs, a.row_magic, a.row_shift);
    magic_for(a.head_vecs, a.head_magic, a.head_shift);
    const uint32_t dtile = direct_tile_vecs(vb), htile = headrun_tile_vecs(vb);
    a.tiles = uint32_t((nvec_max + dtile - 1) / dtile);

    // A view whose heads lie further apart than its tokens (head-major
    // storage) makes the token and head axes swap for real: in wire order a
    // workgroup's writes into it scatter 2*D-byte pieces over all Gb heads,
    // and the chip has every head's stream open at once.  Scatters into such
    // views run as head runs instead: a workgroup moves TT consecutive
    // tokens of one head (TT * head_vecs <= the head-run tile), consecutive
    // workgroups continue the same head.  Head rows narrower than a cache
    // line would make those runs read partial lines on the wire side, and
    // make wire-order gathers read partial lines of the view; such views go
    // through the LDS transpose, whose tiles touch whole lines on both
    // sides (for a gather, whole wire rows).  Gathers from head-major views
    // with wider head rows stay in wire order, where the scattered side is
    // the reads, which cost little.
    bool head_major = false;
    for (int i = 0; i < nviews; ++i)
        if (views[i].sh > views[i].st)
            head_major = true;
    const bool gather = op == Op::Pack || op == Op::Split;
    // heads per LDS-transpose tile: a gather writes whole wire rows (all Gb
    // heads, one write stream), a scatter the fewest heads that fill a line
    const int64_t gt = gather ? Gb : staged_heads(Gb, d->D);
    const int64_t lds_budget = gather ? kGatherLdsBytes : kScatterLdsBytes;
    const bool narrow = d->D * 2 < kHeadrunMinBytes && gt * a.head_vecs * vb <= lds_budget;
    int64_t tiles = a.tiles;
    if (!head_major || Gb <= 1) {
        // token-major (or one head per row): wire order (direct kernel)
    } else if (narrow) {
        const int64_t lrow_bytes = gt * a.head_vecs * vb;
        // tokens per tile: as many as fit, rounded to whole lines of a head's run
        const int64_t quantum = std::max<int64_t>(1, 128 / (d->D * 2));
        int64_t tt = lds_budget / lrow_bytes;
        if (tt >= quantum)
            tt -= tt % quantum;
        tt = std::min<int64_t>(tt, t_max);
        a.group_heads = uint32_t(gt);
        a.tile_tokens = uint32_t(tt);
        a.tok_tiles = uint32_t((t_max + tt - 1) / tt);
        magic_for(uint32_t(gt * a.head_vecs), a.gv_magic, a.gv_shift);
        magic_for(uint32_t(tt * a.head_vecs), a.tv_magic, a.tv_shift);
        // LDS column swizzle: g = the largest power of two dividing the row
        // (in vectors), at most one sweep of the 64 four-byte banks; rows
        // t and t + sweep/g start on the same bank, so the swizzle changes
        // every sweep/g tokens.
        const int64_t sweep = 256 / vb;
        int64_t g = 1;
        while (g < sweep && (gt * a.head_vecs) % (2 * g) == 0)
            g *= 2;
        a.swz_mask = uint32_t(g - 1);
        a.swz_shift = 0;
        while ((int64_t(1) << a.swz_shift) < sweep / g)
            ++a.swz_shift;
        pl.lds_bytes = uint32_t(tt * lrow_bytes);
        tiles = (Gb / gt) * int64_t(a.tok_tiles);
    } else if (!gather && a.head_vecs <= htile) {
        const int64_t tt = std::min<int64_t>(htile / a.head_vecs, t_max);
        pl.headrun = true;
        a.tile_tokens = uint32_t(tt);
        a.tok_tiles = uint32_t((t_max + tt - 1) / tt);
        tiles = Gb * int64_t(a.tok_tiles);
    }
    const int64_t planes = (op == Op::Pack || op == Op::Unpack) ? 3 : 1;
    const int64_t grid = int64_t(d->P) * (ce - cb) * planes * tiles;
    if (grid >= (int64_t(1) << 31)) {
        *why = "the launch needs 2^31 workgroups or more";
        return false;
    }
    a.tiles = uint32_t(tiles);
    pl.grid = uint32_t(grid);
    return true;
}

}  // namespace vrl
