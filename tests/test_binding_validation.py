"""The Python binding rejects wrongly shaped, typed or placed tensors with
ValueError before anything reaches the library (CPU only: every case here
fails validation, so no pointer is ever passed on)."""
import pytest
import torch

import sparse_tree_structured_amd as fff

T, d, P, D, h = 8, 64, 2, 3, 48
N = (1 << (D + 1)) - 1
BF = torch.bfloat16


def layer(**over):
    t = dict(x=torch.zeros(T, d, dtype=BF), W_node=torch.zeros(P, N, d, dtype=BF),
             b_node=torch.zeros(P, N, dtype=BF), V_node=torch.zeros(P, N, h, dtype=BF),
             W_out=torch.zeros(P * h, d, dtype=BF))
    t.update(over)
    return t


def fwd(**over):
    L = layer(**{k: v for k, v in over.items() if k in ("x", "W_node", "b_node", "V_node", "W_out")})
    kw = {k: v for k, v in over.items() if k not in L}
    return fff.forward(L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"], **kw)


BAD = [
    ("W_out transposed (nn.Linear layout)", dict(W_out=torch.zeros(d, P * h, dtype=BF)), "W_out"),
    ("W_out short", dict(W_out=torch.zeros(P * h - 1, d, dtype=BF)), "W_out"),
    ("b_node missing a node", dict(b_node=torch.zeros(P, N - 1, dtype=BF)), "b_node"),
    ("b_node flat", dict(b_node=torch.zeros(P * N, dtype=BF)), "b_node"),
    ("V_node with other trees", dict(V_node=torch.zeros(P + 1, N, h, dtype=BF)), "V_node"),
    ("V_node with other nodes", dict(V_node=torch.zeros(P, N + 2, h, dtype=BF)), "V_node"),
    ("W_node not a full tree", dict(W_node=torch.zeros(P, N - 1, d, dtype=BF)), "W_node"),
    ("W_node of another width", dict(W_node=torch.zeros(P, N, d + 1, dtype=BF)), "W_node"),
    ("x three-dimensional", dict(x=torch.zeros(1, T, d, dtype=BF)), "x"),
    ("y too small", dict(y=torch.zeros(T - 1, d, dtype=BF)), "y"),
    ("path_out transposed", dict(path_out=torch.zeros(P, T, dtype=torch.int32)), "path_out"),
    ("workspace two-dimensional", dict(workspace=torch.zeros(4, 4, dtype=torch.uint8)), "workspace"),
]


@pytest.mark.parametrize("what,over,name", BAD, ids=[b[0] for b in BAD])
def test_forward_rejects_shape(what, over, name):
    with pytest.raises(ValueError, match=name):
        fwd(**over)


def test_forward_rejects_dtypes():
    with pytest.raises(ValueError, match="one dtype"):
        fwd(W_out=torch.zeros(P * h, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="one dtype"):
        fwd(y=torch.zeros(T, d, dtype=torch.float32))


def test_forward_rejects_host_tensors():
    # every shape right: the only problem left is that nothing is on a GPU
    with pytest.raises(ValueError, match="GPU"):
        fwd()


def test_other_entry_points_check_shapes():
    L = layer()
    with pytest.raises(ValueError, match="b_node"):
        fff.route(L["x"], L["W_node"], torch.zeros(P, N + 1, dtype=BF), L["V_node"])
    with pytest.raises(ValueError, match="disagree on K"):
        fff.project(torch.zeros(T, P * h, dtype=BF), torch.zeros(d, P * h, dtype=BF))
    with pytest.raises(ValueError, match="y"):
        fff.project(torch.zeros(T, P * h, dtype=BF), L["W_out"], y=torch.zeros(T, d + 1, dtype=BF))
    pr = fff.Pruning()
    with pytest.raises(ValueError, match="W_out"):
        fff.forward_pruned(L["x"], L["W_node"], L["b_node"], L["V_node"],
                           torch.zeros(d, P * h, dtype=BF), pr)
    with pytest.raises(ValueError, match="dy"):
        fff.backward(L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"],
                     torch.zeros(T, d + 1, dtype=BF))
    out = {"dx": torch.zeros(T, d, dtype=BF), "dW_node": torch.zeros(P, N, d),
           "db_node": torch.zeros(P, N), "dV_node": torch.zeros(P, N, h),
           "dW_out": torch.zeros(d, P * h)}
    with pytest.raises(ValueError, match="dW_out"):
        fff.backward(L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"],
                     torch.zeros(T, d, dtype=BF), out=out)
