// Host-side status strings, thread-local error detail and argument checks.

#include "host_common.h"

#include <math.h>
#include <stdio.h>

#include <limits>

namespace sdattn {

namespace {
thread_local std::string g_last_error;
}

sdattn_status fail(sdattn_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

sdattn_status check_problem(const sdattn_problem* p, Problem* out) {
    if (p == nullptr) return fail(SDATTN_ERR_NULL, "problem is NULL");
    if (p->batch < 1 || p->q_heads < 1 || p->kv_heads < 1)
        return fail(SDATTN_ERR_SHAPE, "batch, q_heads and kv_heads must be >= 1");
    if (p->q_heads % p->kv_heads != 0)
        return fail(SDATTN_ERR_SHAPE, "q_heads must be a multiple of kv_heads");
    if (p->seq_len < 0) return fail(SDATTN_ERR_SHAPE, "seq_len must be >= 0");
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(SDATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (p->dtype != SDATTN_F32 && p->dtype != SDATTN_BF16)
        return fail(SDATTN_ERR_DTYPE, "dtype must be SDATTN_F32 or SDATTN_BF16");
    if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale))
        return fail(SDATTN_ERR_SHAPE, "softmax_scale must be finite");
    // every index the kernels form stays within 32-bit grid / row counts
    const double rows = static_cast<double>(p->batch) * p->q_heads * (p->seq_len + 63.0);
    if (rows > 2.0e9) return fail(SDATTN_ERR_SHAPE, "batch * q_heads * seq_len too large");
    // one head's K or V slab (plus a tile of rows past its end) is addressed
    // with 32-bit byte offsets
    const double slab = (p->seq_len + 128.0) * p->head_dim * 4.0;
    if (slab >= 4294901760.0) return fail(SDATTN_ERR_SHAPE, "seq_len * head_dim too large");
    out->B = p->batch;
    out->Hq = p->q_heads;
    out->Hkv = p->kv_heads;
    out->L = p->seq_len;
    out->D = p->head_dim;
    out->dtype = p->dtype;
    out->scale = p->softmax_scale > 0.f ? p->softmax_scale : static_cast<float>(1.0 / sqrt(static_cast<double>(p->head_dim)));
    return SDATTN_OK;
}

int64_t count_from_fraction(double frac, int64_t n) {
    double k = ceil(frac * static_cast<double>(n) - 1e-9);
    if (k < 1.0) k = 1.0;
    if (k > static_cast<double>(n)) k = static_cast<double>(n);
    return static_cast<int64_t>(k);
}

sdattn_status check_blocks(const Problem& pr, int32_t block_q, int32_t block_k,
                           const sdattn_budget* b, BlockPlan* out) {
    if (b == nullptr) return fail(SDATTN_ERR_NULL, "budget is NULL");
    if ((block_q != 64 && block_q != 128) || (block_k != 64 && block_k != 128))
        return fail(SDATTN_ERR_UNSUPPORTED, "block_q and block_k must be 64 or 128");
    out->nqb = (pr.L + block_q - 1) / block_q;
    out->nkb = (pr.L + block_k - 1) / block_k;
    if (out->nkb > kMaxKeyBlocks) {
        char buf[128];
        snprintf(buf, sizeof buf, "ceil(seq_len / block_k) = %d exceeds the selector limit %d", out->nkb, kMaxKeyBlocks);
        return fail(SDATTN_ERR_UNSUPPORTED, buf);
    }
    out->rows = static_cast<int64_t>(pr.B) * pr.Hq * out->nqb;
    const int64_t full = out->rows * out->nkb;
    if (b->kind == SDATTN_BUDGET_TOPK) {
        if (!(b->keep_frac > 0.0 && b->keep_frac <= 1.0))
            return fail(SDATTN_ERR_BUDGET, "keep_frac must be in (0, 1]");
        out->mass = false;
        out->topk = out->nkb > 0 ? count_from_fraction(b->keep_frac, out->nkb) : 0;
        out->max_nnz = out->rows * out->topk;
        out->cap_extra = 0;
    } else if (b->kind == SDATTN_BUDGET_MASS) {
        if (!(b->mass > 0.0 && b->mass <= 1.0)) return fail(SDATTN_ERR_BUDGET, "mass must be in (0, 1]");
        if (!(b->max_mean_density > 0.0 && b->max_mean_density <= 1.0))
            return fail(SDATTN_ERR_BUDGET, "max_mean_density must be in (0, 1]");
        out->mass = true;
        out->topk = 0;
        const int64_t allowed = static_cast<int64_t>(floor(b->max_mean_density * static_cast<double>(full) + 1e-9));
        out->cap_extra = allowed - out->rows;
        int64_t m = allowed > out->rows ? allowed : out->rows;
        out->max_nnz = m < full ? m : full;
    } else {
        return fail(SDATTN_ERR_BUDGET, "unknown budget kind");
    }
    if (out->max_nnz > std::numeric_limits<int32_t>::max())
        return fail(SDATTN_ERR_SHAPE, "number of kept blocks exceeds int32 CSR range");
    return SDATTN_OK;
}

}  // namespace sdattn

extern "C" {

int sdattn_abi_version(void) { return SDATTN_ABI_VERSION; }

const char* sdattn_status_string(sdattn_status s) {
    switch (s) {
        case SDATTN_OK: return "SDATTN_OK";
        case SDATTN_ERR_NULL: return "SDATTN_ERR_NULL";
        case SDATTN_ERR_SHAPE: return "SDATTN_ERR_SHAPE";
        case SDATTN_ERR_DTYPE: return "SDATTN_ERR_DTYPE";
        case SDATTN_ERR_BUDGET: return "SDATTN_ERR_BUDGET";
        case SDATTN_ERR_WORKSPACE: return "SDATTN_ERR_WORKSPACE";
        case SDATTN_ERR_CAPACITY: return "SDATTN_ERR_CAPACITY";
        case SDATTN_ERR_HIP: return "SDATTN_ERR_HIP";
        case SDATTN_ERR_UNSUPPORTED: return "SDATTN_ERR_UNSUPPORTED";
        case SDATTN_ERR_STATE: return "SDATTN_ERR_STATE";
    }
    return "SDATTN_ERR_UNKNOWN";
}

const char* sdattn_last_error(void) { return sdattn::g_last_error.c_str(); }

}  // extern "C"
