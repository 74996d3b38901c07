// Host-only check of the launch planner's kernel choice and tile geometry
// (head_relayout_amd/csrc/vrl_plan.cpp), linked without the kernels: for
// each case it prints the plan and compares it with the rule it should
// follow.  Prints one line per case and exits 0 when every case holds.
//
// The rule: token-major views take the direct kernel; head-major views with
// head rows narrower than a 128-byte line take the LDS transpose (for a
// scatter Gt heads filling a line x as many tokens as fit 8 KiB, for a
// gather the whole group x as many tokens as fit 16 KiB);
// scatters into head-major views with wider rows take head runs (16 tokens
// of one head per workgroup at head_dim 128), gathers from them the direct
// kernel; so does any view whose head row is longer than one tile or whose
// group has one head.
#include "../../head_relayout_amd/csrc/vrl_internal.h"

#include <cstdint>
#include <cstdio>

using namespace vrl;

namespace {

enum Kind { DIRECT, HEADRUN, STAGED };

const char *name(Kind k)
{
    return k == DIRECT ? "direct" : k == HEADRUN ? "head-run" : "staged";
}

struct Case {
    const char *what;
    Op op;
    int32_t P, C;
    int64_t S_l;
    int32_t H, D, chunk_heads;
    bool head_major;
    uintptr_t misalign;  // bytes added to the view pointers
    Kind kind;           // expected kernel
    int64_t tt;          // expected tokens per tile (0: not checked)
    int64_t gt;          // expected heads per tile (staged; 0: not checked)
    int64_t grid;        // expected workgroups (0: not checked)
    int vb;              // expected vector bytes
};

bool run(const Case &k)
{
    const Problem pb{k.P, k.C, k.S_l, k.H, k.D, k.chunk_heads};
    const int64_t G = k.H / k.P, S = int64_t(k.P) * k.S_l, HD = int64_t(k.H) * k.D;
    const bool hside = k.op == Op::Pack || k.op == Op::Merge;
    const int64_t rows = hside ? k.S_l : S, heads = hside ? k.H : G;
    PlanView v[3];
    for (int i = 0; i < 3; ++i) {
        const uintptr_t base = (uintptr_t(i + 1) << 36) + k.misalign;
        if (k.head_major)
            v[i] = PlanView{base, k.D, rows * k.D};
        else if (k.op == Op::Pack)
            v[i] = PlanView{(uintptr_t(1) << 36) + 2 * uintptr_t(i) * HD + k.misalign, 3 * HD, k.D};
        else
            v[i] = PlanView{base, heads * k.D, k.D};
    }
    const int nviews = (k.op == Op::Pack || k.op == Op::Unpack) ? 3 : 1;
    LaunchPlan pl;
    const char *why = nullptr;
    if (!plan_launch(k.op, pb, v, nviews, uintptr_t(1) << 40, 0, k.C, pl, &why)) {
        std::printf("%-44s planning failed: %s\n", k.what, why);
        return false;
    }
    const Kind got = pl.headrun ? HEADRUN : pl.lds_bytes ? STAGED : DIRECT;
    bool ok = got == k.kind && pl.vec_bytes == k.vb;
    if (k.tt && got != DIRECT)
        ok = ok && pl.args.tile_tokens == uint32_t(k.tt);
    if (k.gt && got == STAGED)
        ok = ok && pl.args.group_heads == uint32_t(k.gt);
    if (k.grid)
        ok = ok && pl.grid == uint32_t(k.grid);
    if (got == STAGED) {  // the LDS tile fits the budget and holds whole rows
        const uint32_t gv = pl.args.group_heads * pl.args.head_vecs;
        const bool gather = k.op == Op::Pack || k.op == Op::Split;
        ok = ok && pl.lds_bytes <= (gather ? kGatherLdsBytes : kScatterLdsBytes) &&
             pl.lds_bytes == pl.args.tile_tokens * gv * uint32_t(pl.vec_bytes);
        // the column swizzle is a power-of-two mask dividing the row, so it
        // permutes columns within the row
        const uint32_t m = pl.args.swz_mask;
        ok = ok && (m & (m + 1)) == 0 && gv % (m + 1) == 0 && (m + 1) * uint32_t(pl.vec_bytes) <= 256;
    }
    std::printf("%-44s %-8s vb=%2d tt=%5u gt=%2u grid=%8u lds=%5u %s\n", k.what, name(got), pl.vec_bytes,
                got == DIRECT ? 0u : pl.args.tile_tokens, got == STAGED ? pl.args.group_heads : 0u, pl.grid,
                pl.lds_bytes, ok ? "ok" : "UNEXPECTED");
    return ok;
}

}  // namespace

int main()
{
    // representative shape: P=2, C=4, 27,707 tokens per rank, 56 heads of 128
    const int64_t R = 27707;
    const Case cases[] = {
        // 1 KiB direct tiles: 6,927 tokens x 448 vectors / 64 = 48,489 per (rank, chunk, plane)
        {"pack, fused token-major source", Op::Pack, 2, 4, R, 56, 128, 0, false, 0, DIRECT, 0, 0, 1163736, 16},
        {"unpack, token-major", Op::Unpack, 2, 4, R, 56, 128, 0, false, 0, DIRECT, 0, 0, 1163736, 16},
        {"split, token-major", Op::Split, 2, 4, R, 56, 128, 0, false, 0, DIRECT, 0, 0, 387912, 16},
        {"merge, token-major", Op::Merge, 2, 4, R, 56, 128, 0, false, 0, DIRECT, 0, 0, 387912, 16},
        // 28 heads x 433 token tiles of 16 per (rank, chunk, plane)
        {"unpack into head-major, D=128", Op::Unpack, 2, 4, R, 56, 128, 0, true, 0, HEADRUN, 16, 0, 290976, 16},
        {"merge into head-major, D=128", Op::Merge, 2, 4, R, 56, 128, 0, true, 0, HEADRUN, 16, 0, 96992, 16},
        {"split from head-major, D=128", Op::Split, 2, 4, R, 56, 128, 0, true, 0, DIRECT, 0, 0, 387912, 16},
        {"pack from head-major, D=128", Op::Pack, 2, 4, R, 56, 128, 0, true, 0, DIRECT, 0, 0, 1163736, 16},
        {"unpack into head-major, head chunks", Op::Unpack, 2, 4, R, 56, 128, 1, true, 0, HEADRUN, 16, 0, 0, 16},
        {"unpack into head-major, D=64", Op::Unpack, 2, 4, 2 * R, 56, 64, 0, true, 0, HEADRUN, 32, 0, 0, 16},
        // 126-byte head rows: 2 heads fill a line; 2*63 2-byte vectors per LDS row
        {"unpack into head-major, D=63", Op::Unpack, 2, 3, 20, 4, 63, 0, true, 0, STAGED, 7, 2, 0, 2},
        // 4 heads x 32 B fill a line; 8 vectors per LDS row, 8 KiB scatter tiles -> 64 tokens
        {"unpack into head-major, D=16", Op::Unpack, 2, 4, 8 * R, 56, 16, 0, true, 0, STAGED, 64, 4, 0, 16},
        {"merge into head-major, D=16", Op::Merge, 2, 4, 8 * R, 56, 16, 0, true, 0, STAGED, 64, 4, 0, 16},
        {"unpack into head-major, D=32", Op::Unpack, 2, 4, 4 * R, 56, 32, 0, true, 0, STAGED, 64, 2, 0, 16},
        // gathers: whole wire rows (28 heads); 56 vectors per LDS row -> 18 tokens, rounded to 16
        {"split from head-major, D=16", Op::Split, 2, 4, 8 * R, 56, 16, 0, true, 0, STAGED, 16, 28, 0, 16},
        // 112 vectors per LDS row -> 9 tokens, rounded to 8
        {"pack from head-major, D=32", Op::Pack, 2, 4, 4 * R, 56, 32, 0, true, 0, STAGED, 8, 28, 0, 16},
        {"unpack into head-major, D=8, 5 heads", Op::Unpack, 2, 4, 64, 10, 8, 0, true, 0, STAGED, 0, 5, 0, 16},
        {"unpack into head-major, one head per group", Op::Unpack, 2, 4, 64, 2, 128, 0, true, 0, DIRECT, 0, 0, 0, 16},
        {"unpack into head-major, D=16392", Op::Unpack, 2, 2, 3, 4, 16392, 0, true, 0, DIRECT, 0, 0, 0, 16},
        // narrow vectors: 4 KiB tiles at every width: 16 tokens x 1 KiB rows -> 4 tiles per block
        {"unpack, views 2-byte aligned", Op::Unpack, 2, 4, 64, 8, 128, 0, false, 2, DIRECT, 0, 0, 96, 2},
        {"unpack, views 8-byte aligned", Op::Unpack, 2, 4, 64, 8, 128, 0, false, 8, DIRECT, 0, 0, 96, 8},
        {"unpack into head-major, 4-byte aligned, D=128", Op::Unpack, 2, 4, 64, 8, 128, 0, true, 4, HEADRUN, 16, 0, 0, 4},
    };
    int bad = 0;
    for (const Case &k : cases)
        bad += run(k) ? 0 : 1;
    std::printf("%s: %d of %zu cases as expected\n", bad ? "FAILED" : "plan rules ok",
                int(sizeof(cases) / sizeof(cases[0])) - bad, sizeof(cases) / sizeof(cases[0]));
    return bad ? 1 : 0;
}
