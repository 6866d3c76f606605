// Host fusion pass (dlf_fusion_plan): picks the Conv/MatMul -> BN -> activation chains of a
// graph that become one fused launch, in the three stages of the CANN graph-autofusion
// article (pattern matching, benefit estimation, greedy conflict resolution), with the
// legality checks of the OpenPPL fusion article (§4.1 unique consumer and inference-mode BN,
// §4.2 no broadcast in the epilogue).  Host code only; no HIP call.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/dlfusion.h"
#include "status.h"

namespace {

using dlf::fail;
using dlf::ok;

// Position of an epilogue op in the fused kernel's fixed order (bias/BN -> residual Add ->
// activation -> quantisation); -1 for ops that never join a chain.
int epilogue_stage(int op) {
    switch (op) {
        case DLF_OP_BIAS_ADD: case DLF_OP_BATCHNORM: return 0;
        case DLF_OP_ADD: return 1;
        case DLF_OP_RELU: case DLF_OP_GELU_TANH: case DLF_OP_GELU_ERF: return 2;
        case DLF_OP_QUANT: return 3;
        default: return -1;
    }
}

bool is_contraction(int op) { return op == DLF_OP_CONV || op == DLF_OP_MATMUL || op == DLF_OP_MATMUL_FP8; }

int64_t elem_bytes(int dtype) { return dtype == DLF_F32 ? 4 : dtype == DLF_BF16 ? 2 : 1; }

bool same_shape(const dlf_graph_node& a, const dlf_graph_node& b) {
    if (a.rank != b.rank) return false;
    for (int d = 0; d < a.rank; ++d)
        if (a.shape[d] != b.shape[d]) return false;
    return true;
}

struct Graph {
    const dlf_graph_node* nd;
    int n;
    std::vector<int> n_readers;     // input slots that read each node's tensor
    std::vector<int> first_reader;  // the reader, when there is exactly one slot
    std::vector<int64_t> bytes;     // tensor size
};

// May node `next` (the only reader of the chain's last value) extend the chain?
bool extends(const Graph& g, const std::vector<int>& chain, int next) {
    const dlf_graph_node& head = g.nd[chain.front()];
    const dlf_graph_node& x = g.nd[next];
    const int stage = epilogue_stage(x.op);
    if (stage < 0) return false;
    const int last_stage = chain.size() == 1 ? -1 : epilogue_stage(g.nd[chain.back()].op);
    if (stage <= last_stage) return false;                   // the epilogue order is fixed
    if (!same_shape(x, head)) return false;                  // elementwise on the output
    if (x.op == DLF_OP_BATCHNORM && (x.flags & DLF_NODE_TRAINING)) return false;
    if (x.op == DLF_OP_ADD) {
        if (head.op == DLF_OP_MATMUL_FP8 || x.n_inputs != 2 || x.dtype != head.dtype) return false;
        const int prev = chain.back();
        if ((x.inputs[0] == prev) == (x.inputs[1] == prev)) return false;   // x + x
        const dlf_graph_node& r = g.nd[x.inputs[0] == prev ? x.inputs[1] : x.inputs[0]];
        return same_shape(r, x) && r.dtype == x.dtype;       // a full tensor: no broadcast
    }
    if (x.n_inputs != 1) return false;
    if (x.op == DLF_OP_QUANT) return head.op == DLF_OP_MATMUL_FP8;
    return x.dtype == head.dtype;
}

struct Candidate {
    std::vector<int> ops;
    int64_t saved;
    double net;
};

dlf_status validate(const dlf_graph_node* nodes, int32_t n) {
    for (int i = 0; i < n; ++i) {
        const dlf_graph_node& x = nodes[i];
        if (x.op < DLF_OP_INPUT || x.op > DLF_OP_OTHER)
            return fail(DLF_ERR_INVALID_ARG, "node %d: unknown op %d", i, x.op);
        if (x.n_inputs < 0 || x.n_inputs > 2)
            return fail(DLF_ERR_INVALID_ARG, "node %d: n_inputs must be 0..2", i);
        for (int j = 0; j < x.n_inputs; ++j)
            if (x.inputs[j] < 0 || x.inputs[j] >= i)
                return fail(DLF_ERR_INVALID_ARG, "node %d: input %d is not an earlier node", i, x.inputs[j]);
        if (x.dtype != DLF_F32 && x.dtype != DLF_BF16 && x.dtype != DLF_FP8_E4M3)
            return fail(DLF_ERR_INVALID_ARG, "node %d: unknown dtype %d", i, x.dtype);
        if (x.rank < 0 || x.rank > 4) return fail(DLF_ERR_INVALID_ARG, "node %d: rank must be 0..4", i);
        int64_t e = elem_bytes(x.dtype);
        for (int d = 0; d < x.rank; ++d) {
            if (x.shape[d] < 0) return fail(DLF_ERR_INVALID_ARG, "node %d: negative extent", i);
            if (x.shape[d] > 0 && e > (int64_t(1) << 56) / x.shape[d])
                return fail(DLF_ERR_INVALID_ARG, "node %d: tensor larger than 2^56 bytes", i);
            e *= x.shape[d];
        }
        if (x.flops < 0) return fail(DLF_ERR_INVALID_ARG, "node %d: negative flops", i);
    }
    return DLF_OK;
}

}  // namespace

extern "C" dlf_status dlf_fusion_plan(const dlf_graph_node* nodes, int32_t n_nodes, double ridge,
                                      double overhead_frac, dlf_fusion_group* groups, int32_t capacity,
                                      int32_t* n_groups) {
    if (!n_groups) return fail(DLF_ERR_INVALID_ARG, "n_groups is NULL");
    if (n_nodes < 0 || capacity < 0) return fail(DLF_ERR_INVALID_ARG, "negative count");
    if (n_nodes > 0 && !nodes) return fail(DLF_ERR_INVALID_ARG, "nodes is NULL");
    if (capacity > 0 && !groups) return fail(DLF_ERR_INVALID_ARG, "groups is NULL");
    if (!std::isfinite(ridge) || ridge <= 0.0) return fail(DLF_ERR_INVALID_ARG, "ridge must be finite and > 0");
    if (!std::isfinite(overhead_frac) || overhead_frac < 0.0)
        return fail(DLF_ERR_INVALID_ARG, "overhead_frac must be finite and >= 0");
    if (dlf_status s = validate(nodes, n_nodes); s != DLF_OK) return s;

    Graph g{nodes, n_nodes, std::vector<int>(n_nodes, 0), std::vector<int>(n_nodes, -1),
            std::vector<int64_t>(n_nodes, 0)};
    for (int i = 0; i < n_nodes; ++i) {
        for (int j = 0; j < nodes[i].n_inputs; ++j) {
            const int p = nodes[i].inputs[j];
            g.first_reader[p] = i;
            ++g.n_readers[p];
        }
        int64_t b = elem_bytes(nodes[i].dtype);
        for (int d = 0; d < nodes[i].rank; ++d) b *= nodes[i].shape[d];
        g.bytes[i] = b;
    }

    // stage 1 (every chain prefix that matches) and stage 2 (benefit) together
    std::vector<Candidate> cands;
    for (int c = 0; c < n_nodes; ++c) {
        if (!is_contraction(nodes[c].op)) continue;
        std::vector<int> chain{c};
        int64_t saved = 0, flops = nodes[c].flops;
        for (;;) {
            const int last = chain.back();
            if ((nodes[last].flags & DLF_NODE_OUTPUT) || g.n_readers[last] != 1) break;
            const int next = g.first_reader[last];
            if (!extends(g, chain, next)) break;
            chain.push_back(next);
            saved += 2 * g.bytes[last];     // written once and read back once when unfused
            flops += nodes[next].flops;
            const double overhead = overhead_frac * static_cast<double>(flops);
            const double net = static_cast<double>(saved) - overhead / ridge;
            if (net > 0.0) cands.push_back(Candidate{chain, saved, net});
        }
    }

    // stage 3: greedy conflict resolution
    std::sort(cands.begin(), cands.end(), [](const Candidate& a, const Candidate& b) {
        if (a.net != b.net) return a.net > b.net;
        if (a.ops.front() != b.ops.front()) return a.ops.front() < b.ops.front();
        return a.ops.size() > b.ops.size();
    });
    std::vector<char> taken(n_nodes, 0);
    std::vector<const Candidate*> chosen;
    for (const Candidate& c : cands) {
        bool clash = false;
        for (int op : c.ops) clash = clash || taken[op];
        if (clash) continue;
        for (int op : c.ops) taken[op] = 1;
        chosen.push_back(&c);
    }
    std::sort(chosen.begin(), chosen.end(),
              [](const Candidate* a, const Candidate* b) { return a->ops.front() < b->ops.front(); });

    *n_groups = static_cast<int32_t>(chosen.size());
    if (static_cast<int64_t>(chosen.size()) > capacity)
        return fail(DLF_ERR_INVALID_ARG, "capacity %d is below the %d groups found", capacity,
                    static_cast<int>(chosen.size()));
    for (size_t i = 0; i < chosen.size(); ++i) {
        dlf_fusion_group& out = groups[i];
        out.count = static_cast<int32_t>(chosen[i]->ops.size());
        for (int j = 0; j < 5; ++j) out.nodes[j] = j < out.count ? chosen[i]->ops[j] : -1;
        out.saved_bytes = chosen[i]->saved;
        out.net_benefit = chosen[i]->net;
    }
    return ok();
}
