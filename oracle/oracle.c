/*
 * CPU oracle for the Ulysses sequence<->head relayout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing but the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load or call this library; the device
 * path never routes through it and shares no code with it.
 *
 * What it computes.  The Vflash "Sol-Engine alignment" page (section "What is
 * enabled", and the operation table under it) says the direct relayout
 * kernels replace the materialised stack/permute/contiguous chain (QKV pack)
 * and cat/permute/contiguous chain (returned-head merge) and that every
 * direct output matched the reference element for element.  The exact result
 * therefore has a plain definition: the materialised chains themselves.  This
 * file performs those chains literally, with a minimal strided-view type and
 * the tensor verbs stack / view / narrow / select / permute / contiguous /
 * cat / copy_ over uint16 BF16 bit patterns (values are moved, never
 * converted, so -0, subnormals and NaN payloads survive).
 *
 * It also keeps a byte account of every tensor a chain materialises, so the
 * allocation screen on the same page (pack peak 2,383,245,312 B, merge peak
 * 794,415,104 B at the representative shape: two materialisations each) can
 * be checked against what the chain actually holds live.
 *
 * Layout readings (the pages fix none of these; each is the plainest one):
 *   - chunks split the tokens of a rank; chunk sizes follow the tensor_split
 *     rule (the first S_l mod C chunks get one extra token);
 *   - dest rank d owns heads [d*G, (d+1)*G), G = H / P;
 *   - rank s holds global tokens [s*S_l, (s+1)*S_l);
 *   - the QKV wire buffer is the concatenation over dest of the concatenation
 *     over chunk of [3][T(c)][G][D] blocks (q/k/v, token, head in group, dim);
 *   - the return wire buffer is the same without the q/k/v axis;
 *   - the attention side sees [S][G][D] with global token order.
 *
 * Parallelism: the generic strided copy spreads its rows over OpenMP
 * threads; nothing else is blocked, fused or reordered.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MAXD 8

typedef struct {
    int32_t P, C;
    int64_t s_local;
    int32_t H, D;
} odims;

/* A caller's 3-D view: element strides of its token and head axes; the last
 * (head_dim) axis has unit stride. */
typedef struct {
    uint16_t *ptr;
    int64_t stride_tok, stride_head;
} oview3;

/* Generic strided view (strides in elements). */
typedef struct {
    uint16_t *data;
    int ndim;
    int64_t size[MAXD];
    int64_t stride[MAXD];
} tv;

/* Live/peak bytes of tensors a chain materialised. */
typedef struct {
    int64_t live, peak;
} acct;

static void acct_add(acct *a, int64_t bytes)
{
    a->live += bytes;
    if (a->live > a->peak)
        a->peak = a->live;
}

static int64_t tv_numel(const tv *t)
{
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i)
        n *= t->size[i];
    return n;
}

static tv tv_dense(uint16_t *data, int ndim, const int64_t *size)
{
    tv t;
    memset(&t, 0, sizeof t);
    t.data = data;
    t.ndim = ndim;
    int64_t s = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        t.size[i] = size[i];
        t.stride[i] = s;
        s *= size[i];
    }
    return t;
}

/* torch.narrow */
static tv tv_narrow(tv t, int dim, int64_t start, int64_t len)
{
    t.data += start * t.stride[dim];
    t.size[dim] = len;
    return t;
}

/* tensor.select(dim, i): drops dim. */
static tv tv_select(tv t, int dim, int64_t i)
{
    t.data += i * t.stride[dim];
    for (int k = dim; k + 1 < t.ndim; ++k) {
        t.size[k] = t.size[k + 1];
        t.stride[k] = t.stride[k + 1];
    }
    t.ndim -= 1;
    return t;
}

/* tensor.view splitting one dim of size outer*inner into (outer, inner). */
static tv tv_unflatten(tv t, int dim, int64_t outer, int64_t inner)
{
    tv r = t;
    r.ndim = t.ndim + 1;
    for (int k = 0; k < dim; ++k) {
        r.size[k] = t.size[k];
        r.stride[k] = t.stride[k];
    }
    r.size[dim] = outer;
    r.stride[dim] = t.stride[dim] * inner;
    r.size[dim + 1] = inner;
    r.stride[dim + 1] = t.stride[dim];
    for (int k = dim + 1; k < t.ndim; ++k) {
        r.size[k + 1] = t.size[k];
        r.stride[k + 1] = t.stride[k];
    }
    return r;
}

/* tensor.view merging dims dim and dim+1; only legal when they are
 * adjacent in memory (returns ndim = -1 otherwise). */
static tv tv_flatten2(tv t, int dim)
{
    if (t.stride[dim] != t.size[dim + 1] * t.stride[dim + 1]) {
        t.ndim = -1;
        return t;
    }
    t.size[dim] *= t.size[dim + 1];
    t.stride[dim] = t.stride[dim + 1];
    for (int k = dim + 1; k + 1 < t.ndim; ++k) {
        t.size[k] = t.size[k + 1];
        t.stride[k] = t.stride[k + 1];
    }
    t.ndim -= 1;
    return t;
}

/* tensor.permute(perm) */
static tv tv_permute(tv t, const int *perm)
{
    tv r = t;
    for (int k = 0; k < t.ndim; ++k) {
        r.size[k] = t.size[perm[k]];
        r.stride[k] = t.stride[perm[k]];
    }
    return r;
}

/* dst.copy_(src): same sizes, element by element. */
static void tv_copy(tv dst, tv src)
{
    int nd = src.ndim;
    int64_t inner = nd ? src.size[nd - 1] : 1;
    int64_t rows = 1;
    for (int k = 0; k + 1 < nd; ++k)
        rows *= src.size[k];
    if (inner == 0 || rows == 0)
        return;
    if (nd == 1) {
        /* one long run: spread it over threads in pieces */
        const int64_t piece = 1 << 16, np = (inner + piece - 1) / piece;
#pragma omp parallel for schedule(static)
        for (int64_t p = 0; p < np; ++p) {
            int64_t e0 = p * piece, e1 = e0 + piece < inner ? e0 + piece : inner;
            for (int64_t e = e0; e < e1; ++e)
                dst.data[e * dst.stride[0]] = src.data[e * src.stride[0]];
        }
        return;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t rem = r, so = 0, dof = 0;
        for (int k = nd - 2; k >= 0; --k) {
            int64_t i = rem % src.size[k];
            rem /= src.size[k];
            so += i * src.stride[k];
            dof += i * dst.stride[k];
        }
        const uint16_t *s = src.data + so;
        uint16_t *d = dst.data + dof;
        int64_t ss = nd ? src.stride[nd - 1] : 1, ds = nd ? dst.stride[nd - 1] : 1;
        for (int64_t e = 0; e < inner; ++e)
            d[e * ds] = s[e * ss];
    }
}

static uint16_t *mat_alloc(acct *a, int64_t numel)
{
    acct_add(a, numel * 2);
    uint16_t *p = (uint16_t *)malloc((size_t)(numel > 0 ? numel : 1) * 2);
    return p;
}

static void mat_free(acct *a, uint16_t *p, int64_t numel)
{
    a->live -= numel * 2;
    free(p);
}

/* tensor.contiguous(): a new dense tensor holding src. */
static tv tv_contiguous(acct *a, tv src)
{
    tv d = tv_dense(mat_alloc(a, tv_numel(&src)), src.ndim, src.size);
    tv_copy(d, src);
    return d;
}

/* torch.stack(list, 0) */
static tv tv_stack(acct *a, const tv *parts, int n)
{
    int64_t size[MAXD];
    size[0] = n;
    for (int k = 0; k < parts[0].ndim; ++k)
        size[k + 1] = parts[0].size[k];
    tv out = tv_dense(mat_alloc(a, (int64_t)n * tv_numel(&parts[0])), parts[0].ndim + 1, size);
    for (int i = 0; i < n; ++i)
        tv_copy(tv_select(out, 0, i), parts[i]);
    return out;
}

/* torch.cat(list, 0) */
static tv tv_cat0(acct *a, const tv *parts, int n)
{
    int64_t size[MAXD];
    int64_t rows = 0;
    for (int i = 0; i < n; ++i)
        rows += parts[i].size[0];
    size[0] = rows;
    for (int k = 1; k < parts[0].ndim; ++k)
        size[k] = parts[0].size[k];
    int64_t per_row = 1;
    for (int k = 1; k < parts[0].ndim; ++k)
        per_row *= size[k];
    tv out = tv_dense(mat_alloc(a, rows * per_row), parts[0].ndim, size);
    int64_t at = 0;
    for (int i = 0; i < n; ++i) {
        tv_copy(tv_narrow(out, 0, at, parts[i].size[0]), parts[i]);
        at += parts[i].size[0];
    }
    return out;
}

/* torch.cat(list, dim) */
static tv tv_cat(acct *a, const tv *parts, int n, int dim)
{
    int64_t size[MAXD];
    for (int k = 0; k < parts[0].ndim; ++k)
        size[k] = parts[0].size[k];
    size[dim] = 0;
    for (int i = 0; i < n; ++i)
        size[dim] += parts[i].size[dim];
    int64_t numel = 1;
    for (int k = 0; k < parts[0].ndim; ++k)
        numel *= size[k];
    tv out = tv_dense(mat_alloc(a, numel), parts[0].ndim, size);
    int64_t at = 0;
    for (int i = 0; i < n; ++i) {
        tv_copy(tv_narrow(out, dim, at, parts[i].size[dim]), parts[i]);
        at += parts[i].size[dim];
    }
    return out;
}

/* ---- chunking: torch.tensor_split(tokens, C) sizes ------------------------ */

static int64_t chunk_len(const odims *d, int c)
{
    int64_t base = d->s_local / d->C, extra = d->s_local % d->C;
    return base + (c < extra ? 1 : 0);
}

static int64_t chunk_start(const odims *d, int c)
{
    int64_t at = 0;
    for (int k = 0; k < c; ++k)
        at += chunk_len(d, k);
    return at;
}

/* Element offset of block (x, c) in a wire buffer that concatenates, for x
 * in [0, P) and then c in [0, C), blocks of `per_token` elements per token. */
static int64_t wire_block_start(const odims *d, int x, int c, int64_t per_token)
{
    int64_t at = 0;
    for (int xx = 0; xx < d->P; ++xx)
        for (int cc = 0; cc < d->C; ++cc) {
            if (xx == x && cc == c)
                return at;
            at += chunk_len(d, cc) * per_token;
        }
    return at;
}

static int dims_ok(const odims *d, int c_begin, int c_end)
{
    if (d->P < 1 || d->C < 1 || d->H < 1 || d->D < 1 || d->s_local < 1)
        return 0;
    if (d->H % d->P != 0 || d->C > d->s_local)
        return 0;
    if (c_begin < 0 || c_end > d->C || c_begin >= c_end)
        return 0;
    return 1;
}

static tv view3(const oview3 *v, int64_t rows, int64_t heads, int64_t dim)
{
    tv t;
    memset(&t, 0, sizeof t);
    t.data = v->ptr;
    t.ndim = 3;
    t.size[0] = rows;
    t.size[1] = heads;
    t.size[2] = dim;
    t.stride[0] = v->stride_tok;
    t.stride[1] = v->stride_head;
    t.stride[2] = 1;
    return t;
}

/* ---- the four chains ------------------------------------------------------- */

/*
 * QKV destination pack ("What is enabled": stack/permute/contiguous chain).
 *   X = stack([q, k, v]) over the window's tokens        -> [3][N][H][D]
 *   Xv = X.view(3, N, P, G, D)
 *   for each dest d and chunk c of the window:
 *       packed[block(d, c)] .copy_( Xv[:, chunk c, d] )   -> [3][T(c)][G][D]
 * Materialised: X and the packed output (twice the output at full window).
 */
int oracle_qkv_pack(const odims *d, const oview3 *q, const oview3 *k, const oview3 *v,
                    uint16_t *packed, int c_begin, int c_end, int64_t *peak_bytes)
{
    if (!dims_ok(d, c_begin, c_end) || !q->ptr || !k->ptr || !v->ptr || !packed)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D;
    const int64_t t0 = chunk_start(d, c_begin), n = chunk_start(d, c_end) - t0;
    tv src[3] = {tv_narrow(view3(q, d->s_local, d->H, D), 0, t0, n),
                 tv_narrow(view3(k, d->s_local, d->H, D), 0, t0, n),
                 tv_narrow(view3(v, d->s_local, d->H, D), 0, t0, n)};
    tv X = tv_stack(&a, src, 3);
    tv Xv = tv_unflatten(X, 2, d->P, G); /* [3][N][P][G][D] */
    acct_add(&a, 3 * n * d->H * D * 2);    /* the packed output, window part */
    for (int dd = 0; dd < d->P; ++dd)
        for (int c = c_begin; c < c_end; ++c) {
            int64_t T = chunk_len(d, c);
            tv blk = tv_select(tv_narrow(Xv, 1, chunk_start(d, c) - t0, T), 2, dd);
            int64_t bs[4] = {3, T, G, D};
            tv slot = tv_dense(packed + wire_block_start(d, dd, c, 3 * G * D), 4, bs);
            tv_copy(slot, blk);
        }
    mat_free(&a, X.data, tv_numel(&X));
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * The same pack in its single-permute form, legal when every chunk has the
 * same length T (S_l divisible by C):
 *   stack([q,k,v]).view(3, C, T, P, G, D).permute(3, 1, 0, 2, 4, 5).contiguous()
 */
int oracle_qkv_pack_permute(const odims *d, const oview3 *q, const oview3 *k, const oview3 *v,
                            uint16_t *packed)
{
    if (!dims_ok(d, 0, d->C) || d->s_local % d->C != 0)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D, T = d->s_local / d->C;
    tv src[3] = {view3(q, d->s_local, d->H, D), view3(k, d->s_local, d->H, D),
                 view3(v, d->s_local, d->H, D)};
    tv X = tv_stack(&a, src, 3);                    /* [3][S_l][H][D] */
    tv Y = tv_unflatten(tv_unflatten(X, 1, d->C, T), 3, d->P, G); /* [3][C][T][P][G][D] */
    static const int perm[6] = {3, 1, 0, 2, 4, 5};
    tv Z = tv_permute(Y, perm);                     /* [P][C][3][T][G][D] */
    tv_copy(tv_dense(packed, 6, Z.size), Z);
    mat_free(&a, X.data, tv_numel(&X));
    return 0;
}

/*
 * Receive-side QKV unpack (the compute-stream stage after the inbound wait,
 * listed in the performance guide's profiling section), to BTHD with B = 1:
 *   for each of q, k, v:
 *       Xq = cat([recv[s][c][q] for s for c in window])   -> [N][G][D]
 *       out_q[rows of (s, c)] .copy_( matching rows of Xq )
 */
int oracle_qkv_unpack(const odims *d, const uint16_t *recv, const oview3 *q, const oview3 *k,
                      const oview3 *v, int c_begin, int c_end, int64_t *peak_bytes)
{
    if (!dims_ok(d, c_begin, c_end) || !recv || !q->ptr || !k->ptr || !v->ptr)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D, S = d->P * d->s_local;
    const int W = c_end - c_begin, nparts = d->P * W;
    const oview3 *outs[3] = {q, k, v};
    tv *parts = (tv *)malloc(sizeof(tv) * (size_t)nparts);
    for (int qi = 0; qi < 3; ++qi) {
        int i = 0;
        for (int s = 0; s < d->P; ++s)
            for (int c = c_begin; c < c_end; ++c) {
                int64_t T = chunk_len(d, c);
                int64_t bs[4] = {3, T, G, D};
                tv blk = tv_dense((uint16_t *)recv + wire_block_start(d, s, c, 3 * G * D), 4, bs);
                parts[i++] = tv_select(blk, 0, qi);
            }
        tv Xq = tv_cat0(&a, parts, nparts);
        tv out = view3(outs[qi], S, G, D);
        int64_t at = 0;
        for (int s = 0; s < d->P; ++s)
            for (int c = c_begin; c < c_end; ++c) {
                int64_t T = chunk_len(d, c);
                tv dst = tv_narrow(out, 0, s * d->s_local + chunk_start(d, c), T);
                tv_copy(dst, tv_narrow(Xq, 0, at, T));
                at += T;
            }
        mat_free(&a, Xq.data, tv_numel(&Xq));
    }
    free(parts);
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * Unpack in single-permute form (equal chunks):
 *   recv.view(P, C, 3, T, G, D).permute(2, 0, 1, 3, 4, 5).contiguous()
 *   -> [3][P][C][T][G][D] == [3][S][G][D], then copy_ into q, k, v.
 */
int oracle_qkv_unpack_permute(const odims *d, const uint16_t *recv, const oview3 *q,
                              const oview3 *k, const oview3 *v)
{
    if (!dims_ok(d, 0, d->C) || d->s_local % d->C != 0)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D, T = d->s_local / d->C, S = d->P * d->s_local;
    int64_t rs[6] = {d->P, d->C, 3, T, G, D};
    tv R = tv_dense((uint16_t *)recv, 6, rs);
    static const int perm[6] = {2, 0, 1, 3, 4, 5};
    tv Z = tv_contiguous(&a, tv_permute(R, perm));
    int64_t zs[4] = {3, S, G, D};
    tv Zf = tv_dense(Z.data, 4, zs);
    const oview3 *outs[3] = {q, k, v};
    for (int qi = 0; qi < 3; ++qi)
        tv_copy(view3(outs[qi], S, G, D), tv_select(Zf, 0, qi));
    mat_free(&a, Z.data, tv_numel(&Z));
    return 0;
}

/*
 * Attention-result split ("attention result pack"; one materialisation per
 * call, 94.7 MiB per chunk window at the representative shape):
 *   Ov = O.view(P, S_l, G, D)
 *   for each dest d and chunk c of the window:
 *       send[block(d, c)] .copy_( Ov[d, chunk c] )          -> [T(c)][G][D]
 */
int oracle_attn_split(const odims *d, const oview3 *o, uint16_t *send, int c_begin, int c_end,
                      int64_t *peak_bytes)
{
    if (!dims_ok(d, c_begin, c_end) || !o->ptr || !send)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D;
    tv Ov = tv_unflatten(view3(o, d->P * d->s_local, G, D), 0, d->P, d->s_local);
    for (int dd = 0; dd < d->P; ++dd)
        for (int c = c_begin; c < c_end; ++c)
            acct_add(&a, chunk_len(d, c) * G * D * 2);
    for (int dd = 0; dd < d->P; ++dd)
        for (int c = c_begin; c < c_end; ++c) {
            int64_t T = chunk_len(d, c);
            tv src = tv_narrow(tv_select(Ov, 0, dd), 0, chunk_start(d, c), T);
            int64_t bs[3] = {T, G, D};
            tv_copy(tv_dense(send + wire_block_start(d, dd, c, G * D), 3, bs), src);
        }
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * Returned-head merge ("final unpack"; the cat/permute/contiguous chain):
 *   Y = stack([recv[s] (window tokens, [N][G][D]) for s])  -> [P][N][G][D]
 *   Z = Y.permute(1, 0, 2, 3).contiguous()                 -> [N][P][G][D]
 *   out[window tokens] .copy_( Z.view(N, H, D) )
 * Materialised: Y and Z (twice the output at full window).
 */
int oracle_head_merge(const odims *d, const uint16_t *recv, const oview3 *out, int c_begin,
                      int c_end, int64_t *peak_bytes)
{
    if (!dims_ok(d, c_begin, c_end) || !recv || !out->ptr)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, D = d->D;
    const int64_t t0 = chunk_start(d, c_begin), n = chunk_start(d, c_end) - t0;
    tv *parts = (tv *)malloc(sizeof(tv) * (size_t)d->P);
    for (int s = 0; s < d->P; ++s) {
        /* the window's chunks of source s are adjacent in the wire buffer */
        int64_t bs[3] = {n, G, D};
        parts[s] = tv_dense((uint16_t *)recv + wire_block_start(d, s, c_begin, G * D), 3, bs);
    }
    tv Y = tv_stack(&a, parts, d->P);
    static const int perm[4] = {1, 0, 2, 3};
    tv Z = tv_contiguous(&a, tv_permute(Y, perm));
    tv Zf = tv_flatten2(Z, 1); /* [N][H][D] */
    tv_copy(tv_narrow(view3(out, d->s_local, d->H, D), 0, t0, n), Zf);
    mat_free(&a, Z.data, tv_numel(&Z));
    mat_free(&a, Y.data, tv_numel(&Y));
    free(parts);
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * The sequence-head exchange (all-to-all on the collective stream): block
 * (r, c) of sender s becomes block (s, c) of receiver r.  `which` 0 is the
 * QKV exchange (3 planes per token), 1 the attention-result return.
 * send[i] / recv[i] are rank i's wire buffers.
 */
int oracle_exchange(const odims *d, int which, uint16_t *const *send, uint16_t *const *recv)
{
    if (!dims_ok(d, 0, d->C) || (which != 0 && which != 1))
        return -1;
    const int64_t G = d->H / d->P, D = d->D;
    const int64_t per_token = (which == 0 ? 3 : 1) * G * D;
    for (int s = 0; s < d->P; ++s)
        for (int r = 0; r < d->P; ++r)
            for (int c = 0; c < d->C; ++c) {
                int64_t n = chunk_len(d, c) * per_token;
                int64_t sz[1] = {n};
                tv_copy(tv_dense(recv[r] + wire_block_start(d, s, c, per_token), 1, sz),
                        tv_dense(send[s] + wire_block_start(d, r, c, per_token), 1, sz));
            }
    return 0;
}

/* ---- head-chunked layout ----------------------------------------------------
 *
 * The other reading of the four-chunk layout: the C chunks split each
 * destination's head group (Gc = G / C heads per chunk) instead of its
 * tokens.  Wire blocks then hold all S_l tokens: the QKV buffer is
 * [P][C][3][S_l][Gc][D] and the return buffer [P][C][S_l][Gc][D].  Windows
 * select head chunks.
 */

static int hc_ok(const odims *d, int c_begin, int c_end)
{
    if (d->P < 1 || d->C < 1 || d->H < 1 || d->D < 1 || d->s_local < 1)
        return 0;
    if (d->H % d->P != 0 || (d->H / d->P) % d->C != 0)
        return 0;
    if (c_begin < 0 || c_end > d->C || c_begin >= c_end)
        return 0;
    return 1;
}

/* Element offset of block (x, c): blocks of `blk` elements, x-major. */
static int64_t hc_block_start(const odims *d, int x, int c, int64_t blk)
{
    int64_t at = 0;
    for (int xx = 0; xx < d->P; ++xx)
        for (int cc = 0; cc < d->C; ++cc) {
            if (xx == x && cc == c)
                return at;
            at += blk;
        }
    return at;
}

/*
 * QKV pack, head-chunked:
 *   X = stack([q, k, v])                     -> [3][S_l][H][D]
 *   Xv = X.view(3, S_l, P, C, Gc, D)
 *   packed[block(d, c)] .copy_( Xv[:, :, d, c] )   -> [3][S_l][Gc][D]
 */
int oracle_qkv_pack_hc(const odims *d, const oview3 *q, const oview3 *k, const oview3 *v,
                       uint16_t *packed, int c_begin, int c_end, int64_t *peak_bytes)
{
    if (!hc_ok(d, c_begin, c_end) || !q->ptr || !k->ptr || !v->ptr || !packed)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, Gc = G / d->C, D = d->D, S_l = d->s_local;
    tv src[3] = {view3(q, S_l, d->H, D), view3(k, S_l, d->H, D), view3(v, S_l, d->H, D)};
    tv X = tv_stack(&a, src, 3);
    tv Xv = tv_unflatten(tv_unflatten(X, 2, d->P, G), 3, d->C, Gc); /* [3][S_l][P][C][Gc][D] */
    acct_add(&a, (int64_t)d->P * (c_end - c_begin) * 3 * S_l * Gc * D * 2);
    for (int dd = 0; dd < d->P; ++dd)
        for (int c = c_begin; c < c_end; ++c) {
            tv blk = tv_select(tv_select(Xv, 2, dd), 2, c); /* [3][S_l][Gc][D] */
            int64_t bs[4] = {3, S_l, Gc, D};
            tv_copy(tv_dense(packed + hc_block_start(d, dd, c, 3 * S_l * Gc * D), 4, bs), blk);
        }
    mat_free(&a, X.data, tv_numel(&X));
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * QKV unpack, head-chunked: per plane q,
 *   Y_s = cat([recv[s][c][q] for c in window], dim=1)   -> [S_l][W*Gc][D]
 *   Xq  = cat([Y_s for s], dim=0)                       -> [S][W*Gc][D]
 *   out_q[:, window heads] .copy_( Xq )
 */
int oracle_qkv_unpack_hc(const odims *d, const uint16_t *recv, const oview3 *q, const oview3 *k,
                         const oview3 *v, int c_begin, int c_end, int64_t *peak_bytes)
{
    if (!hc_ok(d, c_begin, c_end) || !recv || !q->ptr || !k->ptr || !v->ptr)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, Gc = G / d->C, D = d->D, S_l = d->s_local, S = d->P * S_l;
    const int W = c_end - c_begin;
    const oview3 *outs[3] = {q, k, v};
    tv *chunks = (tv *)malloc(sizeof(tv) * (size_t)W);
    tv *ranks = (tv *)malloc(sizeof(tv) * (size_t)d->P);
    for (int qi = 0; qi < 3; ++qi) {
        for (int s = 0; s < d->P; ++s) {
            for (int c = c_begin; c < c_end; ++c) {
                int64_t bs[4] = {3, S_l, Gc, D};
                tv blk = tv_dense((uint16_t *)recv + hc_block_start(d, s, c, 3 * S_l * Gc * D), 4, bs);
                chunks[c - c_begin] = tv_select(blk, 0, qi);
            }
            ranks[s] = tv_cat(&a, chunks, W, 1);
        }
        tv Xq = tv_cat(&a, ranks, d->P, 0);
        for (int s = 0; s < d->P; ++s)
            mat_free(&a, ranks[s].data, tv_numel(&ranks[s]));
        tv_copy(tv_narrow(view3(outs[qi], S, G, D), 1, c_begin * Gc, W * Gc), Xq);
        mat_free(&a, Xq.data, tv_numel(&Xq));
    }
    free(chunks);
    free(ranks);
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * Attention-result split, head-chunked:
 *   Ov = O.view(P, S_l, C, Gc, D)
 *   send[block(d, c)] .copy_( Ov[d, :, c] )          -> [S_l][Gc][D]
 */
int oracle_attn_split_hc(const odims *d, const oview3 *o, uint16_t *send, int c_begin, int c_end,
                         int64_t *peak_bytes)
{
    if (!hc_ok(d, c_begin, c_end) || !o->ptr || !send)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, Gc = G / d->C, D = d->D, S_l = d->s_local;
    tv Ov = tv_unflatten(tv_unflatten(view3(o, d->P * S_l, G, D), 0, d->P, S_l), 2, d->C, Gc);
    acct_add(&a, (int64_t)d->P * (c_end - c_begin) * S_l * Gc * D * 2);
    for (int dd = 0; dd < d->P; ++dd)
        for (int c = c_begin; c < c_end; ++c) {
            tv src = tv_select(tv_select(Ov, 0, dd), 1, c); /* [S_l][Gc][D] */
            int64_t bs[3] = {S_l, Gc, D};
            tv_copy(tv_dense(send + hc_block_start(d, dd, c, S_l * Gc * D), 3, bs), src);
        }
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/*
 * Returned-head merge, head-chunked:
 *   Y = stack([recv[s][window chunks] ([W][S_l][Gc][D]) for s])  -> [P][W][S_l][Gc][D]
 *   Z = Y.permute(2, 0, 1, 3, 4).contiguous()                    -> [S_l][P][W][Gc][D]
 *   out.view(S_l, P, C, Gc, D)[:, :, window] .copy_( Z )
 */
int oracle_head_merge_hc(const odims *d, const uint16_t *recv, const oview3 *out, int c_begin,
                         int c_end, int64_t *peak_bytes)
{
    if (!hc_ok(d, c_begin, c_end) || !recv || !out->ptr)
        return -1;
    acct a = {0, 0};
    const int64_t G = d->H / d->P, Gc = G / d->C, D = d->D, S_l = d->s_local;
    const int W = c_end - c_begin;
    tv *parts = (tv *)malloc(sizeof(tv) * (size_t)d->P);
    for (int s = 0; s < d->P; ++s) {
        int64_t bs[4] = {W, S_l, Gc, D};
        parts[s] = tv_dense((uint16_t *)recv + hc_block_start(d, s, c_begin, S_l * Gc * D), 4, bs);
    }
    tv Y = tv_stack(&a, parts, d->P);
    static const int perm[5] = {2, 0, 1, 3, 4};
    tv Z = tv_contiguous(&a, tv_permute(Y, perm));
    tv O = tv_unflatten(tv_unflatten(view3(out, S_l, d->H, D), 1, d->P, G), 2, d->C, Gc);
    tv_copy(tv_narrow(O, 2, c_begin, W), Z);
    mat_free(&a, Z.data, tv_numel(&Z));
    mat_free(&a, Y.data, tv_numel(&Y));
    free(parts);
    if (peak_bytes)
        *peak_bytes = a.peak;
    return 0;
}

/* Exchange of head-chunked wire buffers: block (r, c) of sender s becomes
 * block (s, c) of receiver r. */
int oracle_exchange_hc(const odims *d, int which, uint16_t *const *send, uint16_t *const *recv)
{
    if (!hc_ok(d, 0, d->C) || (which != 0 && which != 1))
        return -1;
    const int64_t Gc = d->H / d->P / d->C;
    const int64_t blk = (which == 0 ? 3 : 1) * d->s_local * Gc * d->D;
    for (int s = 0; s < d->P; ++s)
        for (int r = 0; r < d->P; ++r)
            for (int c = 0; c < d->C; ++c) {
                int64_t sz[1] = {blk};
                tv_copy(tv_dense(recv[r] + hc_block_start(d, s, c, blk), 1, sz),
                        tv_dense(send[s] + hc_block_start(d, r, c, blk), 1, sz));
            }
    return 0;
}

void oracle_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int oracle_threads(void)
{
    return omp_get_max_threads();
}
