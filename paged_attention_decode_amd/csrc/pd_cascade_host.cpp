// Host side of cascade decode: detection of a shared page span, the split of
// the page table into a shared level and a per-request level, and the row
// layout that lets one merge finish a mixed batch.
//
// Method: mlxcel cascade-attention doc.
//  * Detection (section on how sharing is found): sharing is read off the CSR
//    page table positionally -- page i of two requests is shared when both
//    hold the same pool row there.  Candidates are grouped by their first
//    page; a group's shared span is the run of leading positions on which all
//    of its members agree; the group that saves the most page reads,
//    span * (members - 1), is chosen.  A request whose window starts inside
//    its first page is not a candidate; the span stops one page short of
//    every member's last page (level 0 declares its pages full); a span
//    below the minimum page count, or a group below the minimum member
//    count, does not cascade.
//  * Split and merge (sections on the two levels and the one merge): level 0
//    is the shared span attended once with the members' heads stacked;
//    level 1 is every request's own pages -- a member's pages after the span,
//    a non-member's whole list; each request's merge group holds its level-0
//    rows (members only) and then its level-1 rows, so a non-member's group
//    is its own rows alone.

#include <algorithm>
#include <string>
#include <vector>

#include "pd_internal.h"

using namespace pd;

namespace {

struct Group {
    int32_t first_page;
    std::vector<int32_t> members;   // ascending request order
};

}  // namespace

extern "C" int paged_cascade_detect(int32_t batch, const int32_t *indptr, const int32_t *indices,
                                    const int32_t *first_page_offset, int32_t min_shared_pages,
                                    int32_t min_members, int32_t *member_req,
                                    int32_t *num_members, int32_t *shared_pages)
{
    if (!indptr || !first_page_offset || !member_req || !num_members || !shared_pages ||
        (batch > 0 && indptr[batch] > 0 && !indices))
        return fail(PD_E_NULL, "paged_cascade_detect: null pointer");
    if (batch < 0 || min_shared_pages < 1 || min_members < 2)
        return fail(PD_E_ARG, "paged_cascade_detect: need batch >= 0, min_shared_pages >= 1, "
                              "min_members >= 2");
    *num_members = 0;
    *shared_pages = 0;

    // candidates, ordered by (first page, request): equal first pages are
    // then adjacent and each group lists its members in request order
    std::vector<std::pair<int32_t, int32_t>> cand;
    for (int32_t r = 0; r < batch; ++r) {
        const int32_t p = indptr[r + 1] - indptr[r];
        if (p >= 1 && first_page_offset[r] == 0) cand.emplace_back(indices[indptr[r]], r);
    }
    std::sort(cand.begin(), cand.end());

    int64_t best_score = -1;
    int32_t best_leader = -1;
    std::vector<int32_t> best_members;
    int32_t best_span = 0;
    for (size_t i = 0; i < cand.size();) {
        size_t j = i;
        Group g{cand[i].first, {}};
        while (j < cand.size() && cand[j].first == g.first_page) g.members.push_back(cand[j++].second);
        i = j;
        const int32_t m = int32_t(g.members.size());
        if (m < min_members) continue;
        int32_t cap = INT32_MAX;
        for (int32_t r : g.members) cap = std::min(cap, indptr[r + 1] - indptr[r] - 1);
        const int32_t *lead = indices + indptr[g.members[0]];
        int32_t span = 0;
        while (span < cap) {
            bool same = true;
            for (int32_t r : g.members)
                if (indices[indptr[r] + span] != lead[span]) {
                    same = false;
                    break;
                }
            if (!same) break;
            ++span;
        }
        if (span < min_shared_pages) continue;
        const int64_t score = int64_t(span) * (m - 1);
        // ties go to the group whose first member comes first in the batch
        if (score > best_score || (score == best_score && g.members[0] < best_leader)) {
            best_score = score;
            best_leader = g.members[0];
            best_members = g.members;
            best_span = span;
        }
    }
    if (best_score < 0) return PD_OK;
    std::copy(best_members.begin(), best_members.end(), member_req);
    *num_members = int32_t(best_members.size());
    *shared_pages = best_span;
    return PD_OK;
}

// Checks that member_req names distinct requests in ascending order that hold
// the shared span, and returns -1 for non-members / the member index.
static int member_index(int32_t batch, const int32_t *indptr, const int32_t *indices,
                        const int32_t *first_page_offset, const int32_t *member_req,
                        int32_t num_members, int32_t shared_pages, std::vector<int32_t> &midx,
                        const char *who)
{
    if (num_members < 1 || shared_pages < 1)
        return fail(PD_E_ARG, std::string(who) + ": need num_members >= 1 and shared_pages >= 1");
    midx.assign(size_t(batch), -1);
    for (int32_t m = 0; m < num_members; ++m) {
        const int32_t r = member_req[m];
        if (r < 0 || r >= batch || (m > 0 && r <= member_req[m - 1]))
            return fail(PD_E_ARG, std::string(who) + ": member_req must be ascending requests");
        if (first_page_offset[r] != 0 || indptr[r + 1] - indptr[r] < shared_pages + 1)
            return fail(PD_E_ARG, std::string(who) +
                                      ": a member must start on a page boundary and hold more "
                                      "pages than the span");
        for (int32_t i = 0; i < shared_pages; ++i)
            if (indices[indptr[r] + i] != indices[indptr[member_req[0]] + i])
                return fail(PD_E_ARG, std::string(who) + ": members do not share the span");
        midx[size_t(r)] = m;
    }
    return PD_OK;
}

extern "C" int paged_cascade_split(int32_t batch, int32_t page_size, const int32_t *indptr,
                                   const int32_t *indices, const int32_t *last_page_len,
                                   const int32_t *first_page_offset, const int32_t *member_req,
                                   int32_t num_members, int32_t shared_pages, int32_t *indices0,
                                   int32_t *indptr1, int32_t *indices1, int32_t *last_page_len1,
                                   int32_t *first_page_offset1)
{
    if (!indptr || !indices || !last_page_len || !first_page_offset || !member_req ||
        !indices0 || !indptr1 || !last_page_len1 || !first_page_offset1)
        return fail(PD_E_NULL, "paged_cascade_split: null pointer");
    if (batch < 1 || page_size < 1) return fail(PD_E_ARG, "paged_cascade_split: bad sizes");
    std::vector<int32_t> midx;
    const int rc = member_index(batch, indptr, indices, first_page_offset, member_req, num_members,
                               shared_pages, midx, "paged_cascade_split");
    if (rc != PD_OK) return rc;
    if (indptr[batch] - int64_t(num_members) * shared_pages > 0 && !indices1)
        return fail(PD_E_NULL, "paged_cascade_split: null indices1");
    const int32_t *lead = indices + indptr[member_req[0]];
    std::copy(lead, lead + shared_pages, indices0);
    indptr1[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        const int32_t skip = midx[size_t(r)] >= 0 ? shared_pages : 0;
        const int32_t b = indptr[r] + skip, e = indptr[r + 1];
        std::copy(indices + b, indices + e, indices1 + indptr1[r]);
        indptr1[r + 1] = indptr1[r] + (e - b);
        last_page_len1[r] = last_page_len[r];
        first_page_offset1[r] = skip ? 0 : first_page_offset[r];
    }
    return PD_OK;
}

extern "C" int paged_cascade_layout(int32_t batch, const int32_t *member_req, int32_t num_members,
                                    int32_t level0_rows, const int32_t *o_indptr1, int32_t *dst0,
                                    int32_t *dst1, int32_t *o_indptr)
{
    if (!member_req || !o_indptr1 || !dst0 || !o_indptr || (batch > 0 && o_indptr1[batch] > 0 && !dst1))
        return fail(PD_E_NULL, "paged_cascade_layout: null pointer");
    if (batch < 1 || num_members < 1 || level0_rows < 1)
        return fail(PD_E_ARG, "paged_cascade_layout: bad sizes");
    std::vector<int32_t> midx(size_t(batch), -1);
    for (int32_t m = 0; m < num_members; ++m) {
        const int32_t r = member_req[m];
        if (r < 0 || r >= batch || (m > 0 && r <= member_req[m - 1]))
            return fail(PD_E_ARG, "paged_cascade_layout: member_req must be ascending requests");
        midx[size_t(r)] = m;
    }
    o_indptr[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        const int32_t own = o_indptr1[r + 1] - o_indptr1[r];
        if (own < 0) return fail(PD_E_INDPTR, "paged_cascade_layout: o_indptr1 not monotone");
        const int32_t lead = midx[size_t(r)] >= 0 ? level0_rows : 0;
        if (midx[size_t(r)] >= 0) dst0[midx[size_t(r)]] = o_indptr[r];
        for (int32_t t = 0; t < own; ++t) dst1[o_indptr1[r] + t] = o_indptr[r] + lead + t;
        o_indptr[r + 1] = o_indptr[r] + lead + own;
    }
    return PD_OK;
}

extern "C" int paged_cascade_merge_layout(int32_t batch, const int32_t *member_req,
                                          int32_t num_members, int32_t members_per_launch,
                                          int32_t level0_rows, int32_t num_qo_heads,
                                          int32_t *l0_desc)
{
    if (!member_req || !l0_desc) return fail(PD_E_NULL, "paged_cascade_merge_layout: null pointer");
    if (batch < 1 || num_members < 1 || members_per_launch < 1 || level0_rows < 1 ||
        num_qo_heads < 1)
        return fail(PD_E_ARG, "paged_cascade_merge_layout: bad sizes");
    if (int64_t(level0_rows) * num_members * num_qo_heads > INT32_MAX)
        return fail(PD_E_ARG, "paged_cascade_merge_layout: level-0 rows exceed int32");
    for (int32_t r = 0; r < batch; ++r) {
        l0_desc[3 * r] = 0;
        l0_desc[3 * r + 1] = 0;
        l0_desc[3 * r + 2] = -1;
    }
    for (int32_t m = 0; m < num_members; ++m) {
        const int32_t r = member_req[m];
        if (r < 0 || r >= batch || (m > 0 && r <= member_req[m - 1]))
            return fail(PD_E_ARG,
                        "paged_cascade_merge_layout: member_req must be ascending requests");
        const int32_t j = m / members_per_launch;            // launch
        const int32_t first_member = j * members_per_launch;
        const int32_t stack = std::min(members_per_launch, num_members - first_member);
        l0_desc[3 * r] = first_member * level0_rows * num_qo_heads;
        l0_desc[3 * r + 1] = stack;
        l0_desc[3 * r + 2] = m - first_member;
    }
    return PD_OK;
}
