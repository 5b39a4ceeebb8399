// Schedule builder: turns a model shape and a CU count into per-CU instruction
// queues plus the layout of every (CU, compute wave) weight stream.
//
// The schedule is computed once per handle on the host and reused by every
// step, as the page "Megakernels: Deleting the Kernel Boundary to Win Back
// Microseconds" describes for its interpreter (section "One launch, one
// interpreter").  Each stage of a layer is split into one tile per CU; a CU's
// queue holds its tiles in stage order, so every instruction depends only on
// instructions of earlier stages and the queues cannot deadlock (check_plan
// simulates this).
#include "mk_plan.h"

#include <algorithm>
#include <cstdio>

namespace mk {

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

int validate_config(const mk_config& c, std::string& err) {
    char buf[256];
    auto bad = [&](const char* what) {
        snprintf(buf, sizeof buf, "invalid config: %s", what);
        err = buf;
        return (int)MK_ERR_INVALID_ARG;
    };
    auto unsup = [&](const char* what) {
        snprintf(buf, sizeof buf, "unsupported shape: %s", what);
        err = buf;
        return (int)MK_ERR_UNSUPPORTED_SHAPE;
    };
    if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 ||
        c.ffn < 1 || c.vocab < 1 || c.batch < 1 || c.max_seq < 1)
        return bad("every dimension must be positive");
    if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0f)) return bad("rms_eps >= 0 and rope_theta > 0 required");
    if (c.n_cus < 0 || c.n_splits < 0 || c.n_chunks < 0) return bad("n_cus, n_splits, n_chunks must be >= 0");
    if (c.n_q_heads % c.n_kv_heads) return unsup("n_kv_heads must divide n_q_heads");
    if (c.head_dim != 64 && c.head_dim != 128) return unsup("head_dim must be 64 or 128");
    int G = c.n_q_heads / c.n_kv_heads;
    if (NW % G) return unsup("n_q_heads / n_kv_heads must divide 8");
    if (c.hidden % 8 || c.ffn % 8) return unsup("hidden and ffn must be multiples of 8");
    if (c.batch > MAX_BATCH) return unsup("batch must be <= 8");
    if ((c.flags & MK_FLAG_FP8_WEIGHTS) && (c.flags & (MK_FLAG_PROFILE | MK_FLAG_TRACE)))
        return unsup("FP8 weights cannot be combined with profiling or tracing");
    if ((c.flags & MK_FLAG_FP8_WEIGHTS) && c.batch > 4) return unsup("FP8 weights take batch <= 4");
    if (c.n_chunks > 16) return unsup("n_chunks must be <= 16");
    if (c.hidden > 16384 || c.ffn > 65536) return unsup("hidden <= 16384 and ffn <= 65536");
    if ((long long)c.n_q_heads * c.head_dim > 16384) return unsup("n_q_heads * head_dim <= 16384");
    if ((long long)c.max_seq > (1LL << 24)) return unsup("max_seq <= 2^24");
    return MK_OK;
}

namespace {

// rows of one row-group: (matrix, row, k0, klen, src_cols)
struct RowRef {
    uint32_t mat, row, k0, klen, cols;
};

struct Builder {
    Plan& p;
    std::vector<std::vector<Inst>> q;  // per CU
    explicit Builder(Plan& plan) : p(plan), q(plan.ncu) {}

    // rows of row-group `rg` of a GEMV op in layer l (n = 1 or 2)
    int rows_of(const Inst& in, uint32_t rg, RowRef out[2]) const {
        const int l = in.layer, D = p.D, half = D / 2, G = p.G;
        const uint32_t base = (uint32_t)l * MATS_PER_LAYER;
        switch (in.op) {
        case OP_RMS_QKV_ROPE: {
            const int PG = (G + 2) * half;
            int g = rg / PG, t = rg % PG;
            uint32_t mat, r;
            if (t < G * half) {
                int head = g * G + t / half, i = t % half;
                mat = base + MAT_WQ;
                r = head * D + i;
            } else if (t < (G + 1) * half) {
                mat = base + MAT_WK;
                r = g * D + (t - G * half);
            } else {
                mat = base + MAT_WV;
                r = g * D + (t - (G + 1) * half);
            }
            out[0] = {mat, r, 0, (uint32_t)p.H, (uint32_t)p.H};
            out[1] = {mat, r + (uint32_t)half, 0, (uint32_t)p.H, (uint32_t)p.H};
            return 2;
        }
        case OP_O_PROJ_RES:
            out[0] = {base + MAT_WO, rg, 0, (uint32_t)(p.Hq * D), (uint32_t)(p.Hq * D)};
            return 1;
        case OP_RMS_UP_GATE: {  // rg0 = CU slot, rg - rg0 = row-group within its share
            const uint32_t r = p.ug_row((int)in.rg0, rg - in.rg0);
            out[0] = {base + MAT_GATE, r, 0, (uint32_t)p.H, (uint32_t)p.H};
            out[1] = {base + MAT_UP, r, 0, (uint32_t)p.H, (uint32_t)p.H};
            return 2;
        }
        case OP_DOWN_RES: {
            int c = in.a;
            uint32_t k0 = p.chunk_begin[c], k1 = p.chunk_begin[c + 1];
            out[0] = {base + MAT_DOWN, rg, k0, k1 - k0, (uint32_t)p.F};
            return 1;
        }
        case OP_RMS_LM_HEAD:
            if (p.lm_pairs) {
                out[0] = {(uint32_t)p.lm_mat(), 2 * rg, 0, (uint32_t)p.H, (uint32_t)p.H};
                out[1] = {(uint32_t)p.lm_mat(), 2 * rg + 1, 0, (uint32_t)p.H, (uint32_t)p.H};
                return 2;
            }
            out[0] = {(uint32_t)p.lm_mat(), rg, 0, (uint32_t)p.H, (uint32_t)p.H};
            return 1;
        default:
            return 0;
        }
    }

    int kunits_of(int op) const {
        switch (op) {
        case OP_O_PROJ_RES: return p.ku_q;
        case OP_DOWN_RES: return p.ku_f;
        default: return p.ku_h;
        }
    }

    // split [0, n) into ncu contiguous tiles starting at CU `first`
    void tiles(uint16_t op, int layer, int n, uint16_t a = 0) {
        for (int t = 0; t < p.ncu; ++t) {
            int r0 = (int)((long long)n * t / p.ncu), r1 = (int)((long long)n * (t + 1) / p.ncu);
            if (r1 > r0) q[t].push_back(Inst{op, (uint16_t)layer, (uint32_t)r0, (uint32_t)(r1 - r0), a, 0});
        }
    }
};

}  // namespace

int build_plan(const mk_config& c, int ncu, Plan& p, std::string& err) {
    int rc = validate_config(c, err);
    if (rc != MK_OK) return rc;
    if (ncu < 1) {
        err = "n_cus must be >= 1";
        return MK_ERR_INVALID_ARG;
    }
    p = Plan();
    p.L = c.n_layers; p.H = c.hidden; p.Hq = c.n_q_heads; p.Hkv = c.n_kv_heads; p.D = c.head_dim;
    p.F = c.ffn; p.V = c.vocab; p.B = c.batch; p.max_seq = c.max_seq; p.G = p.Hq / p.Hkv;
    p.tied = c.tied_embeddings != 0; p.eps = c.rms_eps; p.theta = c.rope_theta;
    p.ncu = ncu;
    // down-projection K-chunks: 2 for 2 to 4 batch rows with F <= 8192 (every GEMV takes the batched
    // path there, and fewer chunk instructions mean fewer instruction boundaries on the critical
    // path), else 4 (at batch 1 a chunk of at most four units keeps the batch-1 GEMV path; with
    // more rows or a wider F, two chunks would take the LDS the weight rings need)
    p.n_chunk = c.n_chunks ? c.n_chunks : (p.B >= 2 && p.B <= 4 && p.F <= 8192 ? 2 : 4);
    if (p.n_chunk > p.F / 8) p.n_chunk = std::max(1, p.F / 8);
    if (c.n_splits) {
        p.n_split = c.n_splits;
    } else {
        // at most one attention unit per CU, and about 64 keys per split or more:
        // a split costs a fixed latency (one 64-key block per wave, a merge) and
        // every extra split adds work to the reduce (measured best at 1K context)
        int by_cu = std::max(1, ncu / (p.B * p.Hkv));
        int by_len = std::max(1, ceil_div(p.max_seq, 64));
        p.n_split = std::min(std::min(by_cu, by_len), 64);
    }
    if (p.n_split > 256) {
        err = "n_splits must be <= 256";
        return MK_ERR_UNSUPPORTED_SHAPE;
    }
    p.fp8 = (c.flags & MK_FLAG_FP8_WEIGHTS) != 0;
    p.epu = p.fp8 ? FP8_UNIT_ELEMS : UNIT_ELEMS;
    p.ku_h = ceil_div(p.H, p.epu);
    p.ku_q = ceil_div(p.Hq * p.D, p.epu);
    int maxc = 0;
    for (int i = 0; i <= p.n_chunk; ++i) {
        // chunk boundaries on multiples of 8 elements
        p.chunk_begin[i] = (int)((long long)(p.F / 8) * i / p.n_chunk) * 8;
        if (i == p.n_chunk) p.chunk_begin[i] = p.F;
        if (i) maxc = std::max(maxc, p.chunk_begin[i] - p.chunk_begin[i - 1]);
    }
    p.ku_f = ceil_div(maxc, p.epu);
    p.lm_pairs = p.V % 2 == 0 && p.B > 1 && !batch1_path(p.B, p.ku_h, p.fp8);
    p.n_stages = p.L * STAGES_PER_LAYER + 1;
    // global row indices (per-row FP8 scales) and the row-group scale table layout
    {
        uint64_t acc = 0;
        p.mat_row_off.assign((size_t)p.n_mats() + 1, 0);
        for (int m = 0; m < p.n_mats(); ++m) {
            uint32_t rows = 0, cols = 0;
            p.mat_shape((uint32_t)m, rows, cols);
            p.mat_row_off[(size_t)m] = (uint32_t)acc;
            acc += rows;
            if (acc > 0xffffffffull) {
                err = "more than 2^32 weight rows";
                return MK_ERR_UNSUPPORTED_SHAPE;
            }
        }
        p.mat_row_off[(size_t)p.n_mats()] = (uint32_t)acc;
        const uint64_t n_pairs = (uint64_t)(p.Hq + 2 * p.Hkv) * p.D / 2;
        p.rgs_off[0] = 0;
        p.rgs_off[1] = (uint32_t)n_pairs;
        p.rgs_off[2] = (uint32_t)(n_pairs + p.H);
        p.rgs_off[3] = (uint32_t)(n_pairs + p.H + p.F);
        p.rgs_stride = (uint32_t)(n_pairs + 2 * (uint64_t)p.H + p.F);
        if ((uint64_t)p.rgs_stride * p.L + p.V > 0x7fffffffull) {
            err = "the row-group scale table exceeds 2^31 entries";
            return MK_ERR_UNSUPPORTED_SHAPE;
        }
    }

    Builder b(p);
    std::vector<std::vector<uint32_t>> stage_pc(ncu, std::vector<uint32_t>(p.n_stages + 1, 0));
    auto mark = [&](int st) {
        for (int cu = 0; cu < ncu; ++cu) stage_pc[cu][st] = (uint32_t)b.q[cu].size();
    };
    const int n_qkv_pairs = (p.Hq + 2 * p.Hkv) * p.D / 2;
    for (int l = 0; l < p.L; ++l) {
        const int st = l * STAGES_PER_LAYER;
        mark(st + 0);
        b.tiles(OP_RMS_QKV_ROPE, l, n_qkv_pairs);
        mark(st + 1);
        // attention units (row, group, split): unit u on CU u % ncu
        int na = p.B * p.Hkv * p.n_split;
        for (int u = 0; u < na; ++u) {
            int s = u % p.n_split, g = (u / p.n_split) % p.Hkv, bb = u / (p.n_split * p.Hkv);
            b.q[u % ncu].push_back(Inst{OP_ATTENTION, (uint16_t)l, (uint32_t)s, 0, (uint16_t)bb, (uint16_t)g});
        }
        mark(st + 2);
        // reduce units (row, head), spread evenly over the CUs
        int nr = p.B * p.Hq;
        for (int u = 0; u < nr; ++u) {
            int cu = (int)((long long)u * ncu / nr);
            b.q[cu].push_back(Inst{OP_ATTN_REDUCE, (uint16_t)l, 0, 0, (uint16_t)(u / p.Hq), (uint16_t)(u % p.Hq)});
        }
        mark(st + 3);
        b.tiles(OP_O_PROJ_RES, l, p.H);
        mark(st + 4);
        // up/gate rows go chunk by chunk: every CU computes its share of
        // K-chunk 0 of the down projection first, then of chunk 1, ..., so a
        // chunk is complete after the matching fraction of the stage instead
        // of after the whole stage, and the down instructions of the early
        // chunks find their inputs ready.  One instruction per CU holds all
        // its shares in that order (every output word carries its own tag,
        // so no instruction boundary is needed between chunks)
        for (int t = 0; t < ncu; ++t) {
            const uint32_t n = p.ug_count(t);
            if (n) b.q[t].push_back(Inst{OP_RMS_UP_GATE, (uint16_t)l, (uint32_t)t, n, 0, 0});
        }
        mark(st + 5);
        // down projection: a CU owns rows [r0, r1) for every K-chunk, one
        // instruction per chunk, each waiting only for its chunk of the SwiGLU output
        for (int t = 0; t < ncu; ++t) {
            int r0 = (int)((long long)p.H * t / ncu), r1 = (int)((long long)p.H * (t + 1) / ncu);
            if (r1 <= r0) continue;
            for (int cch = 0; cch < p.n_chunk; ++cch)
                b.q[t].push_back(Inst{OP_DOWN_RES, (uint16_t)l, (uint32_t)r0, (uint32_t)(r1 - r0), (uint16_t)cch, 0});
        }
    }
    mark(p.L * STAGES_PER_LAYER);
    b.tiles(OP_RMS_LM_HEAD, p.L, p.lm_pairs ? p.V / 2 : p.V);  // layer field unused for the head
    for (auto& qq : b.q)
        for (auto& in : qq)
            if (in.op == OP_RMS_LM_HEAD) in.layer = 0;
    mark(p.n_stages);

    // flatten queues, stage table
    p.queue_begin.assign(ncu + 1, 0);
    for (int cu = 0; cu < ncu; ++cu) p.queue_begin[cu + 1] = p.queue_begin[cu] + (uint32_t)b.q[cu].size();
    p.insts.reserve(p.queue_begin[ncu]);
    for (int cu = 0; cu < ncu; ++cu) p.insts.insert(p.insts.end(), b.q[cu].begin(), b.q[cu].end());
    p.stage_pc.assign((size_t)ncu * (p.n_stages + 1), 0);
    for (int cu = 0; cu < ncu; ++cu)
        for (int st = 0; st <= p.n_stages; ++st) p.stage_pc[(size_t)cu * (p.n_stages + 1) + st] = stage_pc[cu][st];

    // stream sizes and unit offsets at each instruction boundary
    p.unit_off.assign(((size_t)p.queue_begin[ncu] + ncu) * NW, 0);
    p.stream_len.assign((size_t)ncu * NW, 0);
    for (int cu = 0; cu < ncu; ++cu) {
        uint64_t len[NW] = {0};
        const size_t n = b.q[cu].size();
        for (size_t pc = 0; pc <= n; ++pc) {
            for (int w = 0; w < NW; ++w) {
                if (len[w] > 0xffffffffull) {
                    err = "a weight stream exceeds 2^32 units";
                    return MK_ERR_UNSUPPORTED_SHAPE;
                }
                p.unit_off[((size_t)p.queue_begin[cu] + cu + pc) * NW + w] = (uint32_t)len[w];
            }
            if (pc == n) break;
            const Inst& in = b.q[cu][pc];
            RowRef rr[2];
            for (uint32_t i = 0; i < in.nrg && in.op != OP_ATTENTION && in.op != OP_ATTN_REDUCE; ++i) {
                int nrows = b.rows_of(in, in.rg0 + i, rr);
                len[i % NW] += (uint64_t)nrows * b.kunits_of(in.op);
            }
        }
        for (int w = 0; w < NW; ++w) p.stream_len[(size_t)cu * NW + w] = len[w];
    }
    // The loader streams a GEMV instruction's units as unit-rows (unit j of every compute wave at
    // once), as many as the wave with the most units in it needs; the other waves skip the rest.
    // The row count goes into field b of the instruction, so every wave knows where it ends.
    for (int cu = 0; cu < ncu; ++cu) {
        const size_t qb = p.queue_begin[cu];
        for (size_t pc = 0; pc < b.q[cu].size(); ++pc) {
            Inst& in = p.insts[qb + pc];
            if (in.op == OP_ATTENTION || in.op == OP_ATTN_REDUCE) continue;
            uint32_t rows = 0;
            for (int w = 0; w < NW; ++w) {
                const size_t i0 = (qb + cu + pc) * NW + w, i1 = (qb + cu + pc + 1) * NW + w;
                rows = std::max(rows, p.unit_off[i1] - p.unit_off[i0]);
            }
            if (rows > 0xffffu) {
                err = "an instruction holds more than 65535 weight units per wave";
                return MK_ERR_UNSUPPORTED_SHAPE;
            }
            in.b = (uint16_t)rows;
        }
    }
    // A CU's NW streams are interleaved unit by unit: unit k of wave w sits at
    // cu_base + k * NW + w, so the CU's concurrent reads stay inside one
    // advancing window of NW units (HBM row locality).
    p.stream_base.assign((size_t)ncu * NW, 0);
    uint64_t acc = 0;
    for (int cu = 0; cu < ncu; ++cu) {
        uint64_t mx = 0;
        for (int w = 0; w < NW; ++w) mx = std::max(mx, p.stream_len[(size_t)cu * NW + w]);
        for (int w = 0; w < NW; ++w) p.stream_base[(size_t)cu * NW + w] = acc + w;
        acc += mx * NW;
    }
    p.total_units = acc;

    // pack table: one entry per stream row, in stream order
    std::vector<uint64_t> cursor((size_t)ncu * NW, 0);
    for (int cu = 0; cu < ncu; ++cu) {
        for (const Inst& in : b.q[cu]) {
            if (in.op == OP_ATTENTION || in.op == OP_ATTN_REDUCE) continue;
            const uint32_t ku = (uint32_t)b.kunits_of(in.op);
            RowRef rr[2];
            for (uint32_t i = 0; i < in.nrg; ++i) {
                int nrows = b.rows_of(in, in.rg0 + i, rr);
                uint64_t& cur = cursor[(size_t)cu * NW + i % NW];  // unit index within the wave's stream
                // general GEMV path: the two rows of a row-group alternate unit by unit, so that
                // each x slice read from LDS serves both rows
                const bool inter = nrows == 2 && !batch1_path(p.B, (int)ku, p.fp8);
                for (int k = 0; k < nrows; ++k) {
                    const uint64_t first = inter ? cur + k : cur;
                    p.pack.push_back(PackRow{rr[k].mat, rr[k].row, rr[k].k0, rr[k].klen, rr[k].cols, ku,
                                             inter ? 2u : 1u, p.mat_row_off[rr[k].mat] + rr[k].row,
                                             p.stream_base[(size_t)cu * NW + i % NW] + first * NW});
                    if (!inter) cur += ku;
                }
                if (inter) cur += 2 * (uint64_t)ku;
            }
        }
    }
    return MK_OK;
}

void build_rg_scales(const Plan& p, const std::vector<float>& row_scale, std::vector<float>& out) {
    Builder b(const_cast<Plan&>(p));  // rows_of only reads the plan
    out.assign(((size_t)p.rgs_stride * p.L + p.V) * 2, 1.0f);
    const uint16_t ops[4] = {OP_RMS_QKV_ROPE, OP_O_PROJ_RES, OP_RMS_UP_GATE, OP_DOWN_RES};
    const uint32_t counts[4] = {p.rgs_off[1], (uint32_t)p.H, (uint32_t)p.F, (uint32_t)p.H};
    auto fill = [&](const Inst& in, size_t base, uint32_t n) {
        RowRef rr[2];
        for (uint32_t rg = 0; rg < n; ++rg) {
            const int nr = b.rows_of(in, rg, rr);
            for (int k = 0; k < nr; ++k)
                out[(base + rg) * 2 + k] = row_scale[(size_t)p.mat_row_off[rr[k].mat] + rr[k].row];
        }
    };
    for (int l = 0; l < p.L; ++l)
        for (int o = 0; o < 4; ++o) {
            if (ops[o] == OP_RMS_UP_GATE) {  // indexed by row (the instruction's row-groups are not contiguous)
                const size_t base = (size_t)l * p.rgs_stride + p.rgs_off[o];
                for (int r = 0; r < p.F; ++r) {
                    out[(base + r) * 2] = row_scale[(size_t)p.mat_row_off[(size_t)l * MATS_PER_LAYER + MAT_GATE] + r];
                    out[(base + r) * 2 + 1] = row_scale[(size_t)p.mat_row_off[(size_t)l * MATS_PER_LAYER + MAT_UP] + r];
                }
                continue;
            }
            fill(Inst{ops[o], (uint16_t)l, 0, 0, 0, 0}, (size_t)l * p.rgs_stride + p.rgs_off[o], counts[o]);
        }
    fill(Inst{OP_RMS_LM_HEAD, 0, 0, 0, 0, 0}, (size_t)p.L * p.rgs_stride, (uint32_t)(p.lm_pairs ? p.V / 2 : p.V));
}

// ---------------------------------------------------------------- checking --

bool check_plan(const Plan& p, std::string& err, bool check_order) {
    char buf[256];
    const int ncu = p.ncu, L = p.L, B = p.B;
    const int n_pairs = (p.Hq + 2 * p.Hkv) * p.D / 2;
    // --- coverage: every output produced exactly once per step
    std::vector<int> qkv((size_t)L * n_pairs, 0), o((size_t)L * p.H, 0), ug((size_t)L * p.F, 0),
        dn((size_t)L * p.n_chunk * p.H, 0), lm(p.V, 0), at((size_t)L * B * p.Hkv * p.n_split, 0),
        rd((size_t)L * B * p.Hq, 0);
    for (int cu = 0; cu < ncu; ++cu) {
        int last_stage = -1;
        for (uint32_t i = p.queue_begin[cu]; i < p.queue_begin[cu + 1]; ++i) {
            const Inst& in = p.insts[i];
            int stage;
            switch (in.op) {
            case OP_RMS_QKV_ROPE: stage = in.layer * STAGES_PER_LAYER + 0;
                for (uint32_t r = 0; r < in.nrg; ++r) qkv[(size_t)in.layer * n_pairs + in.rg0 + r]++;
                break;
            case OP_ATTENTION: stage = in.layer * STAGES_PER_LAYER + 1;
                at[(((size_t)in.layer * B + in.a) * p.Hkv + in.b) * p.n_split + in.rg0]++;
                break;
            case OP_ATTN_REDUCE: stage = in.layer * STAGES_PER_LAYER + 2;
                rd[((size_t)in.layer * B + in.a) * p.Hq + in.b]++;
                break;
            case OP_O_PROJ_RES: stage = in.layer * STAGES_PER_LAYER + 3;
                for (uint32_t r = 0; r < in.nrg; ++r) o[(size_t)in.layer * p.H + in.rg0 + r]++;
                break;
            case OP_RMS_UP_GATE: stage = in.layer * STAGES_PER_LAYER + 4;
                if (in.rg0 >= (uint32_t)ncu || in.nrg > p.ug_count((int)in.rg0)) {
                    snprintf(buf, sizeof buf, "CU %d: up/gate instruction beyond its CU share", cu);
                    err = buf;
                    return false;
                }
                for (uint32_t r = 0; r < in.nrg; ++r) ug[(size_t)in.layer * p.F + p.ug_row((int)in.rg0, r)]++;
                break;
            case OP_DOWN_RES: stage = in.layer * STAGES_PER_LAYER + 5;
                for (uint32_t r = 0; r < in.nrg; ++r) dn[((size_t)in.layer * p.n_chunk + in.a) * p.H + in.rg0 + r]++;
                break;
            case OP_RMS_LM_HEAD: stage = L * STAGES_PER_LAYER;
                for (uint32_t r = 0; r < in.nrg; ++r) {
                    if (p.lm_pairs) {
                        if (2 * (size_t)(in.rg0 + r) + 1 >= lm.size()) {
                            err = "LM-head row pair beyond the vocabulary";
                            return false;
                        }
                        lm[2 * (size_t)(in.rg0 + r)]++;
                        lm[2 * (size_t)(in.rg0 + r) + 1]++;
                    } else {
                        lm[in.rg0 + r]++;
                    }
                }
                break;
            default:
                snprintf(buf, sizeof buf, "CU %d: unknown opcode %d", cu, in.op);
                err = buf;
                return false;
            }
            if (check_order && stage < last_stage) {
                snprintf(buf, sizeof buf, "CU %d: queue not in stage order at pc %u", cu, i - p.queue_begin[cu]);
                err = buf;
                return false;
            }
            last_stage = stage;
        }
    }
    auto once = [&](const std::vector<int>& v, const char* what) {
        for (size_t i = 0; i < v.size(); ++i)
            if (v[i] != 1) {
                snprintf(buf, sizeof buf, "%s output %zu produced %d times", what, i, v[i]);
                err = buf;
                return false;
            }
        return true;
    };
    if (!once(qkv, "QKV") || !once(at, "attention") || !once(rd, "reduce") || !once(o, "O-proj") ||
        !once(ug, "up/gate") || !once(dn, "down") || !once(lm, "LM head"))
        return false;

    // --- simulation: an instruction runs once every output it reads exists.
    // Counters of completed outputs per (layer, stage[, group]).
    const int PG = (p.G + 2) * p.D / 2;
    std::vector<int> qkv_grp((size_t)L * p.Hkv, 0), at_cnt((size_t)L * B * p.Hkv, 0), rd_cnt(L, 0), o_cnt(L, 0),
        ug_chunk((size_t)L * p.n_chunk, 0), dn_cnt(L, 0);
    std::vector<uint8_t> o_row((size_t)L * p.H, 0), dn_row((size_t)L * p.H, 0);  // dn_row counts chunks done
    auto hin_full = [&](int l) { return l == 0 || (o_cnt[l - 1] == p.H && dn_cnt[l - 1] == p.n_chunk * p.H); };
    auto hin_rows = [&](int l, uint32_t r0, uint32_t r1) {
        if (l == 0) return true;
        for (uint32_t r = r0; r < r1; ++r)
            if (!o_row[(size_t)(l - 1) * p.H + r] || dn_row[(size_t)(l - 1) * p.H + r] != p.n_chunk) return false;
        return true;
    };
    auto chunk_of = [&](int i) {
        int c = 0;
        while (c + 1 < p.n_chunk && i >= p.chunk_begin[c + 1]) ++c;
        return c;
    };
    auto ready = [&](const Inst& in) {
        const int l = in.layer;
        switch (in.op) {
        case OP_RMS_QKV_ROPE: return hin_full(l);
        case OP_ATTENTION: return qkv_grp[(size_t)l * p.Hkv + in.b] == PG;
        case OP_ATTN_REDUCE: return at_cnt[((size_t)l * B + in.a) * p.Hkv + in.b / p.G] == p.n_split;
        case OP_O_PROJ_RES: return rd_cnt[l] == B * p.Hq && hin_rows(l, in.rg0, in.rg0 + in.nrg);
        case OP_RMS_UP_GATE: return o_cnt[l] == p.H;
        case OP_DOWN_RES:
            return ug_chunk[(size_t)l * p.n_chunk + in.a] == p.chunk_begin[in.a + 1] - p.chunk_begin[in.a];
        case OP_RMS_LM_HEAD: return hin_full(L);
        }
        return false;
    };
    auto complete = [&](const Inst& in) {
        const int l = in.layer;
        switch (in.op) {
        case OP_RMS_QKV_ROPE:
            for (uint32_t r = 0; r < in.nrg; ++r) qkv_grp[(size_t)l * p.Hkv + (in.rg0 + r) / PG]++;
            break;
        case OP_ATTENTION: at_cnt[((size_t)l * B + in.a) * p.Hkv + in.b]++; break;
        case OP_ATTN_REDUCE: rd_cnt[l]++; break;
        case OP_O_PROJ_RES:
            o_cnt[l] += in.nrg;
            for (uint32_t r = 0; r < in.nrg; ++r) o_row[(size_t)l * p.H + in.rg0 + r] = 1;
            break;
        case OP_RMS_UP_GATE:
            for (uint32_t r = 0; r < in.nrg; ++r)
                ug_chunk[(size_t)l * p.n_chunk + chunk_of((int)p.ug_row((int)in.rg0, r))]++;
            break;
        case OP_DOWN_RES:
            dn_cnt[l] += in.nrg;
            for (uint32_t r = 0; r < in.nrg; ++r) dn_row[(size_t)l * p.H + in.rg0 + r]++;
            break;
        default: break;
        }
    };
    std::vector<uint32_t> pc(ncu, 0);
    size_t remaining = p.insts.size();
    while (remaining) {
        bool progress = false;
        for (int cu = 0; cu < ncu; ++cu) {
            while (p.queue_begin[cu] + pc[cu] < p.queue_begin[cu + 1]) {
                const Inst& in = p.insts[p.queue_begin[cu] + pc[cu]];
                if (!ready(in)) break;
                complete(in);
                ++pc[cu];
                --remaining;
                progress = true;
            }
        }
        if (!progress) {
            for (int cu = 0; cu < ncu; ++cu)
                if (p.queue_begin[cu] + pc[cu] < p.queue_begin[cu + 1]) {
                    const Inst& in = p.insts[p.queue_begin[cu] + pc[cu]];
                    snprintf(buf, sizeof buf, "deadlock: CU %d blocked at pc %u (op %d, layer %d)", cu, pc[cu], in.op, in.layer);
                    err = buf;
                    return false;
                }
        }
    }
    // --- pack table: every entry reads inside its source matrix and writes inside the buffer
    for (size_t i = 0; i < p.pack.size(); ++i) {
        const PackRow& r = p.pack[i];
        uint32_t rows = 0, cols = 0;
        if (!p.mat_shape(r.mat, rows, cols) || r.src_cols != cols || (uint64_t)r.k0 + r.klen > cols ||
            r.row >= rows || r.kunits == 0 || (uint64_t)r.klen > (uint64_t)r.kunits * p.epu ||
            (r.ustride != 1 && r.ustride != 2) ||
            r.dst_unit + (uint64_t)(r.kunits - 1) * NW * r.ustride >= p.total_units) {
            snprintf(buf, sizeof buf, "pack entry %zu out of bounds (mat %u row %u k0 %u klen %u)", i, r.mat, r.row,
                     r.k0, r.klen);
            err = buf;
            return false;
        }
    }
    // --- stream layout: pack rows tile every stream exactly
    uint64_t units = 0, stream_units = 0;
    for (const PackRow& r : p.pack) units += r.kunits;
    for (uint64_t len : p.stream_len) stream_units += len;
    if (units != stream_units) {
        snprintf(buf, sizeof buf, "pack rows cover %llu units, streams hold %llu", (unsigned long long)units,
                 (unsigned long long)stream_units);
        err = buf;
        return false;
    }
    return true;
}

bool mutate_plan(Plan& p, int mutation) {
    const int ncu = p.ncu;
    std::vector<std::vector<Inst>> q(ncu);
    for (int cu = 0; cu < ncu; ++cu)
        q[cu].assign(p.insts.begin() + p.queue_begin[cu], p.insts.begin() + p.queue_begin[cu + 1]);
    // the first queue that has a place for the defect
    bool done = false;
    for (int cu = 0; cu < ncu && !done; ++cu) {
        std::vector<Inst>& qc = q[cu];
        if (qc.empty()) continue;
        if (mutation == 1) {
            std::vector<Inst>& qb = q[(cu + 1) % ncu];
            qb.insert(qb.begin() + (qb.empty() ? 0 : 1), qc.front());
            done = true;
        } else if (mutation == 2) {
            for (size_t i = 0; i < qc.size() && !done; ++i)
                if (qc[i].op == OP_RMS_UP_GATE) {
                    qc.erase(qc.begin() + i);
                    done = true;
                }
        } else if (mutation == 3) {
            size_t last_dn = qc.size();
            for (size_t i = 0; i < qc.size(); ++i)
                if (qc[i].op == OP_DOWN_RES) last_dn = i;
            if (last_dn + 1 < qc.size()) {
                std::swap(qc[last_dn], qc[last_dn + 1]);
                done = true;
            }
        }
    }
    if (!done) return false;
    p.insts.clear();
    for (int cu = 0; cu < ncu; ++cu) {
        p.queue_begin[cu] = (uint32_t)p.insts.size();
        p.insts.insert(p.insts.end(), q[cu].begin(), q[cu].end());
    }
    p.queue_begin[ncu] = (uint32_t)p.insts.size();
    return true;
}

}  // namespace mk
