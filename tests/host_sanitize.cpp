// Host half of libpkv (page-table lowering, index validation, both planners,
// metadata copy) driven over seeded random and malformed inputs, for a build
// with AddressSanitizer and UndefinedBehaviorSanitizer.  Every input and
// output buffer is a std::vector of exactly the size the call may touch, so a
// read or write past it, an overflow or any other undefined behaviour aborts
// the run.  Results are also checked against a direct statement of the
// lowering formula (slot = page * p + t mod p) and against the calls' own
// status contracts.  Prints one summary line and exits 0 on success.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

std::mt19937_64 rng(20260601);

int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

// Pointer to a vector's data; an empty vector (which owns no storage) gives
// a one-element dummy, so that no call sees a null array of length zero.
int32_t g_dummy[1];
int32_t* ptr(std::vector<int32_t>& v) { return v.empty() ? g_dummy : v.data(); }
const int32_t* ptr(const std::vector<int32_t>& v) { return v.empty() ? g_dummy : v.data(); }

#define REQUIRE(cond)                                                              \
    do {                                                                           \
        if (!(cond)) {                                                             \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                                          \
        }                                                                          \
    } while (0)

struct Table {
    int32_t B = 0, p = 1;
    std::vector<int32_t> page_indptr, pages, lens;
};

// A page table whose requests share leading runs of pages: requests are put
// in a few families that share a random number of whole pages with a parent
// family, then own pages of their own.
Table random_table(int max_b, int max_len) {
    static const int sizes[] = {1, 2, 3, 7, 16, 128};
    Table t;
    t.B = uni(0, max_b);
    t.p = sizes[uni(0, 5)];
    int next_page = 0;
    std::vector<std::vector<int32_t>> fam_pages(4);
    for (auto& f : fam_pages) {
        const int n = uni(0, 6);
        for (int i = 0; i < n; ++i) f.push_back(next_page++);
    }
    t.page_indptr.assign(t.B + 1, 0);
    for (int b = 0; b < t.B; ++b) {
        const int L = uni(0, max_len);
        const int npg = (L + t.p - 1) / t.p;
        const auto& f = fam_pages[uni(0, 3)];
        int shared = uni(0, (int)f.size());
        shared = std::min(shared, L / t.p);   // a partly filled page is never shared
        for (int j = 0; j < npg; ++j) t.pages.push_back(j < shared ? f[j] : next_page++);
        t.lens.push_back(L);
        t.page_indptr[b + 1] = (int32_t)t.pages.size();
    }
    // scatter the physical page numbers
    std::vector<int32_t> perm(next_page);
    for (int i = 0; i < next_page; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    for (auto& x : t.pages) x = perm[x];
    return t;
}

int64_t total_tokens(const Table& t) {
    int64_t s = 0;
    for (int32_t L : t.lens) s += L;
    return s;
}

void check_lowering(const Table& t) {
    const int64_t n = total_tokens(t);
    std::vector<int32_t> ip(t.B + 1), idx(n);
    pkv_status st = pkv_lower_page_table(t.B, t.p, ptr(t.page_indptr), ptr(t.pages), ptr(t.lens), ptr(ip), ptr(idx),
                                         n);
    REQUIRE(st == PKV_OK);
    int64_t pos = 0;
    for (int b = 0; b < t.B; ++b) {
        REQUIRE(ip[b] == pos);
        for (int tk = 0; tk < t.lens[b]; ++tk)
            REQUIRE(idx[pos++] == t.pages[t.page_indptr[b] + tk / t.p] * t.p + tk % t.p);
    }
    REQUIRE(ip[t.B] == pos);
    // one slot short of the output: refused, nothing written past it
    if (n > 0) {
        std::vector<int32_t> small(n - 1);
        st = pkv_lower_page_table(t.B, t.p, t.page_indptr.data(), t.pages.data(), t.lens.data(), ip.data(),
                                  ptr(small), n - 1);
        REQUIRE(st == PKV_ERANGE);
    }
    // validation of the lowered indices, and of one index outside the pool
    int32_t max_slot = -1;
    for (int32_t x : idx) max_slot = std::max(max_slot, x);
    REQUIRE(pkv_validate_indices(ptr(ip), ptr(idx), t.B, (int64_t)max_slot + 1) == PKV_OK);
    if (n > 0) REQUIRE(pkv_validate_indices(ip.data(), idx.data(), t.B, max_slot) == PKV_ERANGE);
    // a request with one page too many is refused
    if (t.B > 0) {
        Table bad = t;
        bad.pages.insert(bad.pages.begin() + bad.page_indptr[1], 0);
        for (int b = 0; b < bad.B; ++b) bad.page_indptr[b + 1] += 1;
        std::vector<int32_t> ip2(bad.B + 1), idx2(n + 1);
        st = pkv_lower_page_table(bad.B, bad.p, bad.page_indptr.data(), bad.pages.data(), bad.lens.data(), ip2.data(),
                                  idx2.data(), n + 1);
        REQUIRE(st == PKV_ERANGE);
    }
}

// Bins of whole requests: exact-size copy, every request once, short buffer refused.
void check_bins(const pkv_plan* plan, const pkv_plan_info& info, int32_t B) {
    if (info.request_bins == 0) {
        int32_t dummy = 0;
        REQUIRE(pkv_plan_request_bins(plan, &dummy, 1) == PKV_EINVAL);
        return;
    }
    const int64_t n = (int64_t)info.request_bins + 1 + B;
    std::vector<int32_t> bins(n);
    REQUIRE(pkv_plan_request_bins(plan, bins.data(), n) == PKV_OK);
    std::vector<int32_t> short_bins(n - 1);
    REQUIRE(pkv_plan_request_bins(plan, short_bins.data(), n - 1) == PKV_ERANGE);
    REQUIRE(bins[0] == 0 && bins[info.request_bins] == B && info.num_splits == 1);
    std::vector<int> seen(B, 0);
    for (int64_t k = info.request_bins + 1; k < n; ++k) {
        REQUIRE(bins[k] >= 0 && bins[k] < B);
        ++seen[bins[k]];
    }
    for (int32_t b = 0; b < B; ++b) REQUIRE(seen[b] == 1);
}

pkv_tuning random_tuning() {
    pkv_tuning tu;
    pkv_tuning_defaults(&tu);
    if (uni(0, 1)) {
        tu.t_dense = uni(1, 4096);
        tu.gate_ratio = uni(0, 8);
        tu.launch_bytes = (int64_t)uni(0, 1 << 24);
        tu.target_workgroups = uni(1, 4096);
        tu.min_split_tokens = uni(1, 512);
        tu.fuse_cascade = uni(0, 64);
        tu.prefix_target_workgroups = uni(1, 2048);
        tu.min_prefix_split_tokens = uni(1, 2048);
        tu.max_heads_per_item = uni(0, 8);
        tu.prefix_placement = uni(0, 1);
        tu.segment_tokens = uni(0, 1) ? uni(0, 300) : 32;
    }
    return tu;
}

void random_heads(pkv_problem& pr) {
    static const int hkv[] = {1, 2, 3, 4, 8};
    static const int grp[] = {1, 2, 4, 8, 3};
    static const int dims[] = {64, 128, 96};
    pr.num_kv_heads = hkv[uni(0, 4)];
    pr.num_q_heads = pr.num_kv_heads * grp[uni(0, 4)];
    pr.head_dim = dims[uni(0, 2)];
    const int pair = uni(0, 3);
    pr.q_dtype = pair == 0 ? PKV_F32 : PKV_BF16;
    pr.kv_dtype = pair == 0 ? PKV_F32 : pair == 3 ? PKV_FP8_E4M3 : PKV_BF16;
}

void check_plan(const Table& t, int* planned) {
    const int64_t n = total_tokens(t);
    std::vector<int32_t> ip(t.B + 1), idx(n);
    REQUIRE(pkv_lower_page_table(t.B, t.p, ptr(t.page_indptr), ptr(t.pages), ptr(t.lens), ptr(ip), ptr(idx), n) ==
            PKV_OK);
    int32_t min_len = INT32_MAX;
    for (int32_t L : t.lens) min_len = std::min(min_len, L);
    for (int rep = 0; rep < 3; ++rep) {
        pkv_problem pr{};
        pr.batch = t.B;
        random_heads(pr);
        pr.page_size = t.p;
        pr.kv_indptr = ptr(ip);
        pr.kv_indices = uni(0, 1) ? ptr(idx) : nullptr;  // lets the planner look for a contiguous prefix
        pr.shared_prefix_len = t.B > 0 ? uni(0, min_len) : 0;
        pr.force_path = uni(-1, 2);
        pkv_tuning tu = random_tuning();
        pkv_plan* plan = nullptr;
        pkv_status st = pkv_plan_create(&pr, uni(0, 1) ? &tu : nullptr, &plan);
        REQUIRE(st == PKV_OK || st == PKV_EINVAL || st == PKV_EUNSUPPORTED);
        REQUIRE((st == PKV_OK) == (plan != nullptr));
        if (plan) {
            pkv_plan_info info;
            REQUIRE(pkv_plan_get_info(plan, &info) == PKV_OK);
            REQUIRE(info.workspace_bytes >= 0 && info.num_splits >= 1);
            REQUIRE(info.metadata_ints == 0);
            int32_t dummy = 0;
            REQUIRE(pkv_plan_metadata(plan, &dummy, 1) == PKV_EINVAL);  // not a grouped plan
            check_bins(plan, info, t.B);
            pkv_plan_destroy(plan);
            ++*planned;
        }
        // a prefix longer than the shortest request is refused
        if (t.B > 0 && min_len < INT32_MAX) {
            pr.shared_prefix_len = min_len + 1;
            plan = nullptr;
            REQUIRE(pkv_plan_create(&pr, nullptr, &plan) != PKV_OK && plan == nullptr);
        }
    }
}

void check_grouped(const Table& t, int* planned, int64_t* meta_ints) {
    for (int rep = 0; rep < 3; ++rep) {
        pkv_problem pr{};
        pr.batch = t.B;
        random_heads(pr);
        pr.page_size = t.p;
        pr.kv_indptr = nullptr;
        pr.shared_prefix_len = 0;
        pr.force_path = uni(-1, 2);
        pkv_tuning tu = random_tuning();
        pkv_plan* plan = nullptr;
        pkv_status st = pkv_plan_create_grouped(&pr, uni(0, 1) ? &tu : nullptr, ptr(t.page_indptr),
                                                ptr(t.pages), ptr(t.lens), &plan);
        REQUIRE(st == PKV_OK || st == PKV_EINVAL || st == PKV_EUNSUPPORTED);
        if (!plan) continue;
        pkv_plan_info info;
        REQUIRE(pkv_plan_get_info(plan, &info) == PKV_OK);
        check_bins(plan, info, t.B);
        std::vector<int32_t> meta(info.metadata_ints);
        REQUIRE(pkv_plan_metadata(plan, ptr(meta), info.metadata_ints) == PKV_OK);
        if (info.metadata_ints > 0) {
            std::vector<int32_t> short_meta(info.metadata_ints - 1);
            REQUIRE(pkv_plan_metadata(plan, ptr(short_meta),
                                      info.metadata_ints - 1) == PKV_ERANGE);
            // the suffix indices plus the groups' runs cover every token once
            const int32_t* sptr = meta.data();
            int64_t own = sptr[t.B];
            REQUIRE(own <= total_tokens(t));
        }
        *meta_ints += info.metadata_ints;
        pkv_plan_destroy(plan);
        ++*planned;
    }
    // a declared prefix is refused by the grouped planner
    pkv_problem pr{};
    pr.batch = t.B;
    pr.num_q_heads = 8;
    pr.num_kv_heads = 2;
    pr.head_dim = 128;
    pr.q_dtype = pr.kv_dtype = PKV_BF16;
    pr.page_size = t.p;
    pr.shared_prefix_len = 1;
    pr.force_path = -1;
    pkv_plan* plan = nullptr;
    REQUIRE(pkv_plan_create_grouped(&pr, nullptr, ptr(t.page_indptr), ptr(t.pages), ptr(t.lens), &plan) ==
            PKV_EINVAL);
}

// The checked library's checks (host.cpp), on exact-size copies of what a
// step's kernels would read: the arrays the plan was made from pass, and a
// changed indptr, a slot or page outside the pool, a short page list or a
// broken prefix run is refused.
void check_step_checks(const Table& t, int* checked) {
    const int64_t n = total_tokens(t);
    std::vector<int32_t> ip(t.B + 1), idx(n);
    REQUIRE(pkv_lower_page_table(t.B, t.p, ptr(t.page_indptr), ptr(t.pages), ptr(t.lens), ptr(ip), ptr(idx), n) ==
            PKV_OK);
    int32_t max_page = -1, min_len = INT32_MAX;
    for (int32_t x : t.pages) max_page = std::max(max_page, x);
    for (int32_t L : t.lens) min_len = std::min(min_len, L);
    const int64_t num_pages = max_page + 1, num_slots = num_pages * t.p;
    pkv_problem pr{};
    pr.batch = t.B;
    pr.num_q_heads = 8;
    pr.num_kv_heads = 2;
    pr.head_dim = 128;
    pr.q_dtype = pr.kv_dtype = PKV_BF16;
    pr.page_size = t.p;
    pr.kv_indptr = ptr(ip);
    pr.kv_indices = uni(0, 1) ? ptr(idx) : nullptr;
    pr.shared_prefix_len = t.B > 0 ? uni(0, min_len) : 0;
    pr.force_path = uni(-1, 2);
    pkv_plan* plan = nullptr;
    if (pkv_plan_create(&pr, nullptr, &plan) != PKV_OK) return;
    const pkv_plan& pl = *plan;
    std::vector<int32_t> ip2 = ip;
    REQUIRE(pkv::check_step_indptr(pl, ptr(ip2)) == PKV_OK);
    if (t.B > 0) {
        ip2[uni(0, t.B)] += 1;
        REQUIRE(pkv::check_step_indptr(pl, ptr(ip2)) == PKV_EINVAL);
    }
    REQUIRE(pkv::check_slots(ptr(idx), n, num_slots) == PKV_OK);
    if (n > 0) {
        std::vector<int32_t> bad = idx;
        const int64_t at = uni(0, (int)n - 1);
        bad[at] = (int32_t)num_slots;
        REQUIRE(pkv::check_slots(ptr(bad), n, num_slots) == PKV_ERANGE);
        bad[at] = -1;
        REQUIRE(pkv::check_slots(ptr(bad), n, num_slots) == PKV_ERANGE);
    }
    // the prefix pass's slots: request 0's first prefix_tokens
    if (pl.path != PKV_PATH_PAGED && pl.prefix_tokens > 0) {
        std::vector<int32_t> pre(idx.begin(), idx.begin() + pl.prefix_tokens);
        REQUIRE(pkv::check_prefix_slots(pl, ptr(pre), num_slots) == PKV_OK);
        if (pl.prefix_base >= 0) {
            REQUIRE(pkv::check_prefix_slots(pl, ptr(pre), pl.prefix_base + pl.prefix_tokens - 1) == PKV_ERANGE);
            pre[uni(0, pl.prefix_tokens - 1)] += 1;  // no longer the planned run
            REQUIRE(pkv::check_prefix_slots(pl, ptr(pre), num_slots) == PKV_EINVAL);
        } else {
            pre[uni(0, pl.prefix_tokens - 1)] = (int32_t)num_slots;
            REQUIRE(pkv::check_prefix_slots(pl, ptr(pre), num_slots) == PKV_ERANGE);
        }
    }
    // the page table the pages entry reads
    int64_t lo = -1, hi = -1;
    std::vector<int32_t> pip = t.page_indptr;
    REQUIRE(pkv::check_page_indptr(pl, ptr(pip), &lo, &hi) == PKV_OK);
    REQUIRE(0 <= lo && lo <= hi && hi <= (int64_t)t.pages.size());
    REQUIRE(pkv::check_slots(ptr(t.pages) + lo, hi - lo, num_pages) == PKV_OK);
    if (hi > lo) {
        std::vector<int32_t> pg(t.pages.begin() + lo, t.pages.begin() + hi);
        pg[uni(0, (int)(hi - lo) - 1)] = (int32_t)num_pages;
        REQUIRE(pkv::check_slots(ptr(pg), hi - lo, num_pages) == PKV_ERANGE);
    }
    for (int32_t b = 0; b < t.B; ++b) {
        if (t.lens[b] == 0) continue;
        pip = t.page_indptr;  // request b one page short
        for (int32_t c = b + 1; c <= t.B; ++c) pip[c] -= 1;
        REQUIRE(pkv::check_page_indptr(pl, ptr(pip), &lo, &hi) == PKV_ERANGE);
        break;
    }
    if (t.B > 0) {
        pip = t.page_indptr;
        pip[0] = -1;  // a negative first offset
        REQUIRE(pkv::check_page_indptr(pl, ptr(pip), &lo, &hi) == PKV_EINVAL);
    }
    REQUIRE(pkv::check_group_metadata(pl, ptr(idx), num_slots) == PKV_EINVAL);  // not a grouped plan
    pkv_plan_destroy(plan);
    // a grouped step's metadata block
    pr.kv_indptr = nullptr;
    pr.kv_indices = nullptr;
    pr.shared_prefix_len = 0;
    plan = nullptr;
    if (pkv_plan_create_grouped(&pr, nullptr, ptr(t.page_indptr), ptr(t.pages), ptr(t.lens), &plan) != PKV_OK) return;
    pkv_plan_info info;
    REQUIRE(pkv_plan_get_info(plan, &info) == PKV_OK);
    std::vector<int32_t> meta(info.metadata_ints);
    REQUIRE(pkv_plan_metadata(plan, ptr(meta), info.metadata_ints) == PKV_OK);
    REQUIRE(pkv::check_group_metadata(*plan, ptr(meta), num_slots) == PKV_OK);
    if (n > 0) REQUIRE(pkv::check_group_metadata(*plan, ptr(meta), num_slots - 1) == PKV_ERANGE ||
                       *std::max_element(idx.begin(), idx.end()) < num_slots - 1);
    if (info.metadata_ints > 0) {
        meta[uni(0, (int)info.metadata_ints - 1)] ^= 1;
        REQUIRE(pkv::check_group_metadata(*plan, ptr(meta), num_slots) == PKV_EINVAL);
    }
    pkv_plan_destroy(plan);
    ++*checked;
}

void check_malformed() {
    // null pointers, negative sizes, a non-zero first indptr, decreasing indptr
    int32_t ip[3] = {0, 2, 1}, idx[2] = {0, 1}, lens[2] = {2, 0}, out_ip[3];
    REQUIRE(pkv_lower_page_table(-1, 1, ip, idx, lens, out_ip, idx, 2) == PKV_EINVAL);
    REQUIRE(pkv_lower_page_table(2, 0, ip, idx, lens, out_ip, idx, 2) == PKV_EINVAL);
    REQUIRE(pkv_lower_page_table(2, 1, nullptr, idx, lens, out_ip, idx, 2) == PKV_EINVAL);
    REQUIRE(pkv_lower_page_table(2, 1, ip, idx, lens, out_ip, idx, 2) == PKV_EINVAL);  // indptr goes down
    int32_t neg[1] = {-5}, ip1[2] = {0, 1};
    int32_t len1[1] = {1};
    REQUIRE(pkv_lower_page_table(1, 1, ip1, neg, len1, out_ip, idx, 2) == PKV_ERANGE);  // negative page
    int32_t huge[1] = {INT32_MAX / 4};
    REQUIRE(pkv_lower_page_table(1, 16, ip1, huge, len1, out_ip, idx, 2) == PKV_ERANGE);  // slot overflow
    REQUIRE(pkv_validate_indices(nullptr, idx, 1, 4) == PKV_EINVAL);
    REQUIRE(pkv_validate_indices(ip, idx, 2, 4) == PKV_EINVAL);
    pkv_problem pr{};
    pkv_plan* plan = nullptr;
    REQUIRE(pkv_plan_create(nullptr, nullptr, &plan) == PKV_EINVAL);
    REQUIRE(pkv_plan_create(&pr, nullptr, nullptr) == PKV_EINVAL);
    pr.batch = 1;
    pr.num_q_heads = 8;
    pr.num_kv_heads = 3;  // not a divisor
    pr.head_dim = 128;
    pr.q_dtype = pr.kv_dtype = PKV_BF16;
    pr.page_size = 1;
    pr.kv_indptr = ip1;
    REQUIRE(pkv_plan_create(&pr, nullptr, &plan) == PKV_EINVAL);
    pr.num_kv_heads = 2;
    pkv_tuning tu;
    pkv_tuning_defaults(&tu);
    tu.target_workgroups = 0;
    REQUIRE(pkv_plan_create(&pr, &tu, &plan) == PKV_EINVAL);
    REQUIRE(pkv_plan_get_info(nullptr, nullptr) == PKV_EINVAL);
    pkv_plan_destroy(nullptr);
    for (int s = -8; s <= 1; ++s) REQUIRE(pkv_status_string(s) != nullptr);
    pkv_tuning_defaults(nullptr);
    REQUIRE(pkv_version() != nullptr);
}

}  // namespace

int main(int argc, char** argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
    int planned = 0, grouped = 0, checked = 0;
    int64_t meta_ints = 0;
    check_malformed();
    for (int i = 0; i < cases; ++i) {
        const Table t = random_table(i % 10 == 0 ? 300 : 24, i % 7 == 0 ? 3000 : 260);
        check_lowering(t);
        check_plan(t, &planned);
        check_grouped(t, &grouped, &meta_ints);
        check_step_checks(t, &checked);
    }
    std::printf("host_sanitize ok: %d tables, %d plans, %d grouped plans, %lld metadata ints, %d step checks\n",
                cases, planned, grouped, (long long)meta_ints, checked);
    return 0;
}
